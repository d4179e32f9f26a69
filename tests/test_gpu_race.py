"""Race checks on the GPU: the library built with the race-check switches
(every LDS copy destination filled with NaN just before the copy is issued,
and work-group ids visited in a scrambled order) must give bit for bit what
the default library gives, for every kernel family, and must match the fp64
oracle.  A read that overtakes its copy's wait and barrier, or a copy that
overwrites a slot a slow wave still reads, shows up as NaN or as a changed
bit; a result that depended on the order in which work-groups run shows up
as a changed bit."""

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import (LSE_TOL, check_lse, custom, device_inputs, from_device,
                               grad_bound, lib, log_case, max_abs, to_device, torch_cuda)

pytestmark = pytest.mark.gpu


def _debug_lib(fa):
    return fa.load_debug_library()


def _fwd_bwd(fa, torch, cfg, dev, backward=True):
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=cfg.causal,
                        seqlens_k=dev["lengths"])
    out = [o, lse]
    if backward:
        out += list(fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=cfg.scale,
                                causal=cfg.causal, seqlens_k=dev["lengths"]))
    torch.cuda.synchronize()
    return out


def _both(fa, torch, fn):
    ref = fn()
    with fa.library(_debug_lib(fa)):
        got = fn()
    return ref, got


def _assert_bitwise(ref, got, names):
    for name, a, b in zip(names, ref, got):
        assert not (b.float().isnan().any().item() if b.is_floating_point() else False), \
            f"{name}: NaN under the race-check build"
        assert a.shape == b.shape and a.dtype == b.dtype
        assert a.view(-1).view(torch_int(a)).equal(b.view(-1).view(torch_int(b))), \
            f"{name}: differs from the default library"


def torch_int(t):
    import torch
    return {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]


CASES = [
    # (config id, overrides, lengths)
    (5, dict(B=2, H=4, N=1000, d=128, causal=True, dtype="bf16"), [700, 1000]),
    (5, dict(B=2, H=3, N=517, d=64, causal=False, dtype="f16"), None),
    (5, dict(B=1, H=8, N=300, d=256, causal=True, dtype="bf16"), None),
    (5, dict(B=2, H=2, N=200, d=128, causal=True, dtype="f32"), [0, 131]),
    (5, dict(B=1, H=16, N=2048, d=128, causal=True, dtype="bf16"), None),
    (5, dict(B=2, H=3, N=333, d=96, causal=True, dtype="bf16"), [333, 200]),
    (5, dict(B=1, H=4, N=290, d=192, causal=False, dtype="f16"), None),
    (5, dict(B=2, H=2, N=230, d=256, causal=True, dtype="f32"), [230, 97]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forward_backward_race_build_is_bit_identical(case):
    torch = torch_cuda()
    fa = lib()
    cid, over, lengths = CASES[case]
    cfg = custom(cid, **over)
    log_case(test="race", **over, lengths=lengths)
    inputs = fi.make_inputs(cfg, seed=70 + case)
    inputs["lengths"] = None if lengths is None else np.array(lengths, np.int32)
    dev = device_inputs(torch, cfg, inputs)
    ref, got = _both(fa, torch, lambda: _fwd_bwd(fa, torch, cfg, dev))
    _assert_bitwise(ref, got, ("o", "lse", "dq", "dk", "dv"))


def test_race_build_matches_the_oracle():
    """The parity check itself, run once on the race-check build."""
    torch = torch_cuda()
    fa = lib()
    cfg = custom(5, B=2, H=4, N=700, d=128, causal=True, dtype="bf16")
    inputs = fi.make_inputs(cfg, seed=91)
    inputs["lengths"] = np.array([450, 700], np.int32)
    dev = device_inputs(torch, cfg, inputs)
    with fa.library(_debug_lib(fa)):
        o, lse, dq, dk, dv = _fwd_bwd(fa, torch, cfg, dev)
    w = {n: fi.widen(inputs[n], "bf16") for n in ("q", "k", "v", "do")}
    ref_o, ref_l = oracle.attention_materialised(w["q"], w["k"], w["v"], cfg.scale, True,
                                                 inputs["lengths"])
    assert max_abs(from_device(o, "bf16"), ref_o) <= 2e-2
    check_lse(lse.cpu().numpy().astype(np.float64), ref_l, *LSE_TOL["bf16"])
    grads = oracle.attention_backward(w["q"], w["k"], w["v"], ref_o, w["do"], ref_l, cfg.scale,
                                      True, inputs["lengths"])
    for got, ref in zip((dq, dk, dv), grads):
        g = from_device(got, "bf16")
        assert np.all(np.abs(g - ref) <= grad_bound(ref, "bf16"))


def test_fp8_decode_and_packed_race_build_is_bit_identical():
    torch = torch_cuda()
    fa = lib()
    # FP8 forward
    cfg = custom(3, B=1, H=8, N=600, dtype="e4m3")
    inputs = fi.make_inputs(cfg, seed=5)
    q, k, v = (torch.from_numpy(inputs[n]).cuda() for n in ("q", "k", "v"))
    d8 = fi.FP8_DESCALE
    fp8 = lambda: list(fa.forward_fp8(q, k, v, d8["q"], d8["k"], d8["v"], scale=cfg.scale,
                                      causal=True))
    ref, got = _both(fa, torch, lambda: [t.clone() for t in fp8()])
    _assert_bitwise(ref, got, ("o8", "lse8"))
    # decode with cached lengths
    dcfg = fi.DECODE
    dinp = fi.make_decode_inputs(dcfg, lengths="zero_then_uniform")
    up = lambda a: to_device(torch, a, "bf16")
    dq_, dk_, dv_ = up(dinp["q"]), up(dinp["k"]), up(dinp["v"])
    lens = torch.from_numpy(dinp["lengths"]).cuda()
    dec = lambda: list(fa.decode(dq_, dk_, dv_, scale=dcfg.scale, seqlens_k=lens))
    ref, got = _both(fa, torch, dec)
    _assert_bitwise(ref, got, ("o_dec", "lse_dec"))
    # packed variable-length batch, forward and backward
    pcfg = custom(5, H=4, N=700, d=128, dtype="bf16")
    plens = fi.packed_lengths(5, 700, seed=3)
    cu = fi.offsets(plens)
    t = {n: to_device(torch, fi.make_packed(pcfg, n, plens, 0), "bf16") for n in ("q", "k", "v", "do")}
    cu_d = torch.from_numpy(cu).cuda()
    mx = int(plens.max())

    def packed():
        o, lse = fa.forward_varlen(t["q"], t["k"], t["v"], cu_d, cu_d, mx, mx, scale=pcfg.scale,
                                   causal=True)
        g = fa.backward_varlen(t["q"], t["k"], t["v"], o, t["do"], lse, cu_d, cu_d, mx, mx,
                               scale=pcfg.scale, causal=True)
        torch.cuda.synchronize()
        return [o, lse, *g]

    ref, got = _both(fa, torch, packed)
    _assert_bitwise(ref, got, ("o_p", "lse_p", "dq_p", "dk_p", "dv_p"))
