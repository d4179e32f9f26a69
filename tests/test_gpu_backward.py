"""Backward parity on the GPU: fa_backward through the C ABI against the fp64
oracle's exact gradients of <dO, O>.

The GPU backward consumes the GPU forward's O and LSE (its own saved state);
the oracle's gradients use its own fp64 forward.  Tolerance: dQ, dK, dV
max-abs <= 5e-2 for bf16 inputs and <= 2e-2 for f16 (fp32 accumulation; f16
rounds P, dS and the outputs 8x finer than bf16, the bound keeps a margin for
the accumulation order) on the training-step workload; <= 1e-4 for fp32 (fp32
throughout: sums of a few hundred products of O(1) terms with relative
rounding 2^-24 each, plus one ulp of |ref| where the gradient is large).  Edge-case shapes can
make a gradient large (with key length 1, dV of key 0 sums dO over every
row), and from |x| = 16 on one bf16 half-ulp alone exceeds 5e-2 (f16 at 2e-2:
from 64; fp32 at 1e-4: from 2048); only there does the bound add one ulp of
|ref| in the format.
"""

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import (G_TOL, LSE_TOL, ULP, check_lse, custom, device_inputs,
                               from_device, grad_bound, half_ulp_threshold, lib, log_case,
                               max_abs, parallel_map, torch_cuda)

pytestmark = pytest.mark.gpu

O_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}


def run_fwd_bwd(torch, cfg, inputs, lengths=None):
    fa = lib()
    dev = device_inputs(torch, cfg, inputs)
    lens = dev["lengths"]
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=cfg.causal,
                        seqlens_k=lens)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=cfg.scale,
                             causal=cfg.causal, seqlens_k=lens)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def oracle_grads(cfg, inputs, heads=None):
    """fp64 forward + backward on the selected (b, h) heads."""
    w = {n: fi.widen(inputs[n], cfg.dtype) for n in ("q", "k", "v", "do")}
    lengths = inputs.get("lengths")
    out = []
    for (b, h) in heads:
        sl = lambda x: x[b:b + 1, h:h + 1]
        lb = None if lengths is None else np.asarray(lengths)[b:b + 1]
        o, lse = oracle.attention_materialised(sl(w["q"]), sl(w["k"]), sl(w["v"]), cfg.scale,
                                               cfg.causal, lb)
        g = oracle.attention_backward(sl(w["q"]), sl(w["k"]), sl(w["v"]), o, sl(w["do"]), lse,
                                      cfg.scale, cfg.causal, lb)
        out.append((o, g))
    return out


def compare_heads(cfg, inputs, o, dq, dk, dv, heads, strict=False):
    worst = 0.0
    for (b, h), (ref_o, (rq, rk, rv)) in zip(heads, oracle_grads(cfg, inputs, heads)):
        got_o = from_device(o[b:b + 1, h:h + 1], cfg.dtype)
        assert max_abs(got_o, ref_o) <= O_TOL[cfg.dtype]
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            g = from_device(got[b:b + 1, h:h + 1], cfg.dtype)
            assert not np.any(np.isnan(g)), name
            err = max_abs(g, ref)
            if strict:
                assert err <= G_TOL[cfg.dtype], f"{name} head {(b, h)} max abs error {err:.3e}"
            else:
                bound = grad_bound(ref, cfg.dtype)
                assert np.all(np.abs(g - ref) <= bound), f"{name} head {(b, h)} err {err:.3e}"
                small = np.abs(ref) < half_ulp_threshold(cfg.dtype, G_TOL[cfg.dtype])
                err = max_abs(g[small], ref[small])
            worst = max(worst, err)
    return worst


@pytest.mark.parametrize("d", [64, 96, 128, 192])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_small_shapes_all_heads(d, causal, dtype):
    torch = torch_cuda()
    for N in (1, 17, 64, 65, 129, 200, 257):
        for lens_kind in ("none", "edges"):
            lengths = None if lens_kind == "none" else np.array([0, 1, N, max(N - 3, 0)], np.int32)
            B = 2 if lengths is None else 4
            cfg = custom(5, B=B, H=2, N=N, d=d, causal=causal, dtype=dtype)
            log_case(test="bwd-small", N=N, d=d, causal=causal, dtype=dtype, lengths=lens_kind)
            inputs = fi.make_inputs(cfg, seed=100 + N)
            inputs["lengths"] = lengths
            o, lse, dq, dk, dv = run_fwd_bwd(torch, cfg, inputs)
            heads = [(b, h) for b in range(B) for h in range(2)]
            compare_heads(cfg, inputs, o, dq, dk, dv, heads)
            if lengths is not None:
                # keys past the length and every key of the empty sequence get zero gradient
                for b in range(B):
                    Lb = int(lengths[b])
                    assert torch.count_nonzero(dk[b, :, Lb:].view(torch.int16)).item() == 0
                    assert torch.count_nonzero(dv[b, :, Lb:].view(torch.int16)).item() == 0
                assert torch.count_nonzero(dq[0].view(torch.int16)).item() == 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_config5_training_step(dtype):
    """Forward O and LSE on all 64 heads, every row; gradients of four whole
    heads at the stated tolerance; gradient invariants on all 64 heads."""
    torch = torch_cuda()
    cfg = custom(5, dtype=dtype)
    log_case(test="config5", shape=cfg.shape, dtype=dtype)
    inputs = fi.make_inputs(cfg)
    o, lse, dq, dk, dv = run_fwd_bwd(torch, cfg, inputs)
    for t in (o, dq, dk, dv):
        assert not torch.isnan(t).any().item()
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    chunk = 512
    jobs = [(b, h, r0) for (b, h) in heads for r0 in range(0, cfg.N, chunk)]

    def run(job):
        b, h, r0 = job
        q, k, v = (fi.widen(inputs[n][b, h], dtype) for n in ("q", "k", "v"))
        return oracle.attention_rows(q, k, v, np.arange(r0, min(cfg.N, r0 + chunk)), cfg.scale,
                                     True)

    refs = parallel_map(run, jobs)
    o_host = from_device(o, dtype)
    lse_host = lse.cpu().numpy().astype(np.float64)
    worst_o = worst_l = 0.0
    for (b, h, r0), (ref_o, ref_l) in zip(jobs, refs):
        rows = slice(r0, r0 + ref_o.shape[0])
        worst_o = max(worst_o, max_abs(o_host[b, h, rows], ref_o))
        worst_l = max(worst_l, check_lse(lse_host[b, h, rows], ref_l, *LSE_TOL[dtype]))
    assert worst_o <= O_TOL[dtype], f"O max abs error {worst_o:.3e}"
    print(f"config5 {dtype} forward, all 64 heads x 8192 rows: O max abs err {worst_o:.3e}, "
          f"LSE {worst_l:.3e}", flush=True)
    worst = compare_heads(cfg, inputs, o, dq, dk, dv, [(0, 0), (0, 31), (1, 0), (1, 17)],
                          strict=True)
    print(f"config5 {dtype} grads max abs err {worst:.3e}", flush=True)
    # invariants on all 64 heads: every row of dS sums to zero, so sum_j dK_j = 0;
    # sum_j dV_j = sum_i dO_i (every causal row sees key 0); dQ of row 0 is 0.
    # Bound: each 16-bit output carries at most a half-ulp rounding.
    u = ULP[dtype]
    dk64 = dk.double()
    assert (dk64.sum(dim=2).abs() <= dk64.abs().sum(dim=2) * u + 1e-2).all().item()
    do_sum = torch.from_numpy(fi.widen(inputs["do"], dtype).sum(axis=2)).cuda()
    dv64 = dv.double()
    assert ((dv64.sum(dim=2) - do_sum).abs() <= dv64.abs().sum(dim=2) * u + 1e-2).all().item()
    assert dq[:, :, 0].float().abs().max().item() <= 1e-2


def test_backward_is_deterministic():
    torch = torch_cuda()
    cfg = custom(5, B=1, H=3, N=700)
    inputs = fi.make_inputs(cfg, seed=8)
    r1 = run_fwd_bwd(torch, cfg, inputs)
    r2 = run_fwd_bwd(torch, cfg, inputs)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_config1_fp32_backward_every_head():
    """The fp32 workload (one head, N=256, d=64) with dO, causal and not."""
    torch = torch_cuda()
    for causal in (False, True):
        cfg = custom(1, causal=causal)
        log_case(test="config1-bwd", shape=cfg.shape, causal=causal)
        inputs = fi.make_inputs(cfg, with_grad=True, seed=21)
        o, lse, dq, dk, dv = run_fwd_bwd(torch, cfg, inputs)
        worst = compare_heads(cfg, inputs, o, dq, dk, dv, [(0, 0)], strict=True)
        print(f"config1 fp32 causal={causal} grads max abs err {worst:.3e}", flush=True)


def test_fp32_backward_phases_match_the_single_call():
    torch = torch_cuda()
    fa = lib()
    cfg = custom(1, B=2, H=3, N=200, d=128, causal=True)
    inputs = fi.make_inputs(cfg, with_grad=True, seed=4)
    dev = device_inputs(torch, cfg, inputs)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=True)
    g1 = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=cfg.scale, causal=True)
    g2 = fa.backward_phases(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=cfg.scale,
                            causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_head_dim_256_backward(dtype):
    """d = 256: four waves per work-group, one per SIMD, in the 16-bit
    kernels; in the fp32 dK/dV kernel four waves share 32 keys and split the
    feature dimension (partial S and dP added through LDS)."""
    torch = torch_cuda()
    for N in (1, 65, 200):
        for causal in (False, True):
            lengths = np.array([0, 1, N, max(N - 3, 0)], np.int32) if N > 1 else None
            B = 2 if lengths is None else 4
            cfg = custom(5, B=B, H=2, N=N, d=256, causal=causal, dtype=dtype)
            log_case(test="bwd-d256", N=N, causal=causal, dtype=dtype)
            inputs = fi.make_inputs(cfg, seed=300 + N)
            inputs["lengths"] = lengths
            o, lse, dq, dk, dv = run_fwd_bwd(torch, cfg, inputs)
            heads = [(b, h) for b in range(B) for h in range(2)]
            compare_heads(cfg, inputs, o, dq, dk, dv, heads)
