"""Parity on the GPU for Nq query rows against Nk keys (Nq != Nk): the
forward and the backward through the C ABI against the fp64 oracle, causal
(query i sees keys j <= i + Nk - Nq) and not, with and without key lengths,
for every element format.

Tolerances are those of the square problems: O <= 2e-2 (bf16), 5e-3 (f16),
1e-5 (fp32); gradients <= 5e-2, 2e-2, 1e-4 plus one ulp of |ref| in the
format; LSE <= 1e-3 + 1e-5 |LSE| (16-bit) or 1e-5 (fp32); rows that see no
key give O == 0 and LSE == -inf exactly, keys that no query sees get zero
gradients.
"""

import dataclasses

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import (LSE_TOL, check_lse, from_device, grad_bound, lib, log_case,
                               max_abs, to_device, torch_cuda)

pytestmark = pytest.mark.gpu

O_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}

SHAPES = [(1, 300), (7, 129), (65, 300), (200, 64), (300, 65), (129, 1), (64, 256)]


def rect_inputs(dtype, B, H, Nq, Nk, d, seed):
    cfg = dataclasses.replace(fi.CONFIGS[5], B=B, H=H, N=Nq, d=d, dtype=dtype)
    t = {n: fi.make_tensor(cfg, n, seed, N=(Nq if n in ("q", "do") else Nk)) for n in "qkv"}
    t["do"] = fi.make_tensor(cfg, "do", seed, N=Nq)
    return cfg, t


def run(torch, dtype, t, scale, causal, lengths, backward):
    fa = lib()
    dev = {n: to_device(torch, t[n], dtype) for n in t}
    lens = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=scale, causal=causal, seqlens_k=lens)
    grads = None
    if backward:
        grads = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=scale,
                            causal=causal, seqlens_k=lens)
    torch.cuda.synchronize()
    return o, lse, grads


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rectangular_forward_and_backward(dtype, d, causal):
    torch = torch_cuda()
    for Nq, Nk in SHAPES:
        for lens_kind in ("none", "edges"):
            lengths = None if lens_kind == "none" else np.array([0, 1, Nk, max(Nk - 3, 0)],
                                                               np.int32)
            B = 2 if lengths is None else 4
            log_case(test="rect", dtype=dtype, d=d, causal=causal, Nq=Nq, Nk=Nk,
                     lengths=lens_kind)
            cfg, t = rect_inputs(dtype, B, 2, Nq, Nk, d, seed=Nq * 1000 + Nk)
            o, lse, (dq, dk, dv) = run(torch, dtype, t, cfg.scale, causal, lengths, True)
            w = {n: fi.widen(t[n], dtype) for n in t}
            ref_o, ref_l = oracle.attention_materialised(w["q"], w["k"], w["v"], cfg.scale,
                                                         causal, lengths)
            got_o = from_device(o, dtype)
            assert max_abs(got_o, ref_o) <= O_TOL[dtype]
            check_lse(lse.cpu().numpy().astype(np.float64), ref_l, *LSE_TOL[dtype])
            assert np.all(got_o[np.isneginf(ref_l)] == 0.0)
            rq, rk, rv = oracle.attention_backward(w["q"], w["k"], w["v"], ref_o, w["do"], ref_l,
                                                   cfg.scale, causal, lengths)
            for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
                g = from_device(got, dtype)
                assert not np.any(np.isnan(g)), name
                bound = grad_bound(ref, dtype)
                assert np.all(np.abs(g - ref) <= bound), \
                    f"{name} Nq={Nq} Nk={Nk} err {max_abs(g, ref):.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rectangular_d256_backward(dtype):
    torch = torch_cuda()
    for Nq, Nk in ((33, 150), (150, 40)):
        log_case(test="rect-d256-bwd", dtype=dtype, Nq=Nq, Nk=Nk)
        cfg, t = rect_inputs(dtype, 2, 2, Nq, Nk, 256, seed=Nq * 7 + Nk)
        o, lse, (dq, dk, dv) = run(torch, dtype, t, cfg.scale, True, None, True)
        w = {n: fi.widen(t[n], dtype) for n in t}
        ref_o, ref_l = oracle.attention_materialised(w["q"], w["k"], w["v"], cfg.scale, True)
        rq, rk, rv = oracle.attention_backward(w["q"], w["k"], w["v"], ref_o, w["do"], ref_l,
                                               cfg.scale, True)
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            g = from_device(got, dtype)
            assert np.all(np.abs(g - ref) <= grad_bound(ref, dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rectangular_d256_forward(dtype):
    torch = torch_cuda()
    for Nq, Nk in ((33, 300), (300, 100)):
        for causal in (False, True):
            log_case(test="rect-d256", dtype=dtype, Nq=Nq, Nk=Nk, causal=causal)
            cfg, t = rect_inputs(dtype, 2, 2, Nq, Nk, 256, seed=Nq + Nk)
            o, lse, _ = run(torch, dtype, t, cfg.scale, causal, None, False)
            w = {n: fi.widen(t[n], dtype) for n in t}
            ref_o, ref_l = oracle.attention_materialised(w["q"], w["k"], w["v"], cfg.scale,
                                                         causal)
            assert max_abs(from_device(o, dtype), ref_o) <= O_TOL[dtype]
            check_lse(lse.cpu().numpy().astype(np.float64), ref_l, *LSE_TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_side_empty(dtype):
    """Queries without keys: O = 0, LSE = -inf, dQ = 0.  Keys without
    queries: dK = dV = 0."""
    torch = torch_cuda()
    fa = lib()
    log_case(test="rect-empty", dtype=dtype)
    cfg, t = rect_inputs(dtype, 2, 3, 50, 1, 64, seed=3)
    dev = {n: to_device(torch, t[n], dtype) for n in t}
    k0 = dev["k"][:, :, :0].contiguous()
    o, lse = fa.forward(dev["q"], k0, k0, causal=True)
    dq, dk, dv = fa.backward(dev["q"], k0, k0, o, dev["do"], lse, causal=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0 and torch.isneginf(lse).all().item()
    assert torch.count_nonzero(dq).item() == 0 and dk.numel() == 0
    q0 = dev["q"][:, :, :0].contiguous()
    kk = to_device(torch, fi.make_tensor(cfg, "k", 4, N=40), dtype)
    o0 = q0.clone()
    lse0 = torch.empty((2, 3, 0), dtype=torch.float32, device=q0.device)
    dq0, dk0, dv0 = fa.backward(q0, kk, kk, o0, q0, lse0)
    torch.cuda.synchronize()
    assert dk0.shape == kk.shape and torch.count_nonzero(dk0).item() == 0
    assert torch.count_nonzero(dv0).item() == 0
