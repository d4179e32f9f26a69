"""Parity on the GPU for packed batches of variable-length sequences: the
forward and the backward through the C ABI against the fp64 oracle (each
sequence its own problem), for every element format, and bit-for-bit
against the padded entry points called on one sequence at a time.

Tolerances are those of the padded problems: O <= 2e-2 (bf16), 5e-3 (f16),
1e-5 (fp32); gradients <= 5e-2, 2e-2, 1e-4 plus one ulp of |ref| in the
format; LSE <= 1e-3 + 1e-5 |LSE| (16-bit) or 1e-5 (fp32).  Rows that see no
key give O == 0 and LSE == -inf exactly; rows that belong to no sequence
keep what the caller put there.
"""

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import (LSE_TOL, check_lse, custom, from_device, grad_bound, lib,
                               log_case, max_abs, to_device, torch_cuda)

pytestmark = pytest.mark.gpu

O_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}


def packed_case(dtype, d, lens_q, lens_k, H=2, seed=0):
    cfg = custom(5, d=d, dtype=dtype, H=H)
    t = {n: fi.make_packed(cfg, n, lens_q if n in ("q", "do") else lens_k, seed)
         for n in ("q", "k", "v", "do")}
    return cfg, t


def run_packed(torch, dtype, t, lens_q, lens_k, scale, causal, backward=True):
    fa = lib()
    dev = {n: to_device(torch, t[n], dtype) for n in t}
    cu_q = torch.from_numpy(fi.offsets(lens_q)).cuda()
    cu_k = torch.from_numpy(fi.offsets(lens_k)).cuda()
    mq, mk = int(max(lens_q, default=0)), int(max(lens_k, default=0))
    o, lse = fa.forward_varlen(dev["q"], dev["k"], dev["v"], cu_q, cu_k, mq, mk, scale=scale,
                               causal=causal)
    grads = None
    if backward:
        grads = fa.backward_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cu_q, cu_k,
                                   mq, mk, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse, grads


def check_against_oracle(dtype, t, lens_q, lens_k, scale, causal, o, lse, grads):
    w = {n: fi.widen(t[n], dtype) for n in t}
    cu_q, cu_k = fi.offsets(lens_q), fi.offsets(lens_k)
    ref_o, ref_l = oracle.attention_packed(w["q"], w["k"], w["v"], cu_q, cu_k, scale, causal)
    got_o = from_device(o, dtype)
    assert max_abs(got_o, ref_o) <= O_TOL[dtype]
    check_lse(lse.cpu().numpy().astype(np.float64), ref_l, *LSE_TOL[dtype])
    assert np.all(got_o[np.isneginf(ref_l)] == 0.0)
    if grads is None:
        return
    refs = oracle.attention_backward_packed(w["q"], w["k"], w["v"], ref_o, w["do"], ref_l, cu_q,
                                            cu_k, scale, causal)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        g = from_device(got, dtype)
        assert not np.any(np.isnan(g)), name
        bound = grad_bound(ref, dtype)
        assert np.all(np.abs(g - ref) <= bound), f"{name} err {max_abs(g, ref):.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_forward_and_backward(dtype, d, causal):
    """Self-attention lengths (an empty sequence, one of the maximum length,
    the rest uniform) and cross lengths (queries both fewer and more than
    keys), spanning several tiles with ragged tails."""
    torch = torch_cuda()
    lens = fi.packed_lengths(6, 300, seed=d)
    cross_q = np.array([0, 5, 300, 129, 1, 64], np.int32)
    cross_k = np.array([7, 0, 64, 300, 257, 1], np.int32)
    for kind, lq, lk in (("self", lens, lens), ("cross", cross_q, cross_k)):
        log_case(test="packed", dtype=dtype, d=d, causal=causal, kind=kind, lq=list(lq),
                 lk=list(lk))
        cfg, t = packed_case(dtype, d, lq, lk, seed=int(lq.sum()))
        o, lse, grads = run_packed(torch, dtype, t, lq, lk, cfg.scale, causal)
        check_against_oracle(dtype, t, lq, lk, cfg.scale, causal, o, lse, grads)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_head_dim_256(dtype):
    torch = torch_cuda()
    lq = np.array([40, 0, 150, 1], np.int32)
    lk = np.array([150, 33, 150, 90], np.int32)
    for causal in (False, True):
        log_case(test="packed-d256", dtype=dtype, causal=causal)
        cfg, t = packed_case(dtype, 256, lq, lk, seed=11)
        o, lse, grads = run_packed(torch, dtype, t, lq, lk, cfg.scale, causal)
        check_against_oracle(dtype, t, lq, lk, cfg.scale, causal, o, lse, grads)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_is_bitwise_the_padded_call_per_sequence(dtype):
    """A packed sequence runs the same tiles as the padded entry point on that
    sequence alone, so results agree bit for bit (forward and backward),
    including sequences of 8192 rows at the benchmark's head dimension."""
    torch = torch_cuda()
    fa = lib()
    lens = np.array([8192, 3000, 1, 777], np.int32) if dtype == "bf16" else \
        np.array([2048, 300, 1, 777], np.int32)
    log_case(test="packed-vs-padded", dtype=dtype, lens=list(lens))
    cfg, t = packed_case(dtype, 128, lens, lens, H=2, seed=5)
    o, lse, (dq, dk, dv) = run_packed(torch, dtype, t, lens, lens, cfg.scale, True)
    cu = fi.offsets(lens)
    for b, n in enumerate(lens):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        one = {name: to_device(torch, np.ascontiguousarray(t[name][None, :, sl]), dtype)
               for name in t}
        o1, l1 = fa.forward(one["q"], one["k"], one["v"], scale=cfg.scale, causal=True)
        g1 = fa.backward(one["q"], one["k"], one["v"], o1, one["do"], l1, scale=cfg.scale,
                         causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[:, sl], o1[0]), f"o of sequence {b}"
        assert torch.equal(lse[:, sl], l1[0]), f"lse of sequence {b}"
        for name, got, ref in (("dq", dq, g1[0]), ("dk", dk, g1[1]), ("dv", dv, g1[2])):
            assert torch.equal(got[:, sl], ref[0]), f"{name} of sequence {b}"


def test_packed_sampled_rows_at_benchmark_scale():
    """Sequences up to 8192 rows, 32 heads, d = 128, causal bf16: sampled
    rows of each sequence against the oracle, one row at a time."""
    torch = torch_cuda()
    lens = np.array([8192, 5000, 2500, 700, 1], np.int32)
    log_case(test="packed-sampled", lens=list(lens))
    cfg, t = packed_case("bf16", 128, lens, lens, H=32, seed=9)
    o, lse, _ = run_packed(torch, "bf16", t, lens, lens, cfg.scale, True, backward=False)
    got_o, got_l = from_device(o, "bf16"), lse.cpu().numpy().astype(np.float64)
    cu = fi.offsets(lens)
    rng = np.random.default_rng(3)
    for b, n in enumerate(lens):
        for h in rng.choice(32, 3, replace=False):
            rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 4)]))
            base = int(cu[b])
            q = fi.widen(t["q"][h, base:base + n], "bf16")
            k = fi.widen(t["k"][h, base:base + n], "bf16")
            v = fi.widen(t["v"][h, base:base + n], "bf16")
            ref_o, ref_l = oracle.attention_rows(q, k, v, rows, cfg.scale, True)
            assert max_abs(got_o[h, base + rows], ref_o) <= O_TOL["bf16"]
            check_lse(got_l[h, base + rows], ref_l, *LSE_TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_outside_every_sequence_are_left_alone(dtype):
    """Offsets that leave a gap and a tail: those rows keep the caller's
    values in o, lse, dq, dk and dv; a sequence without queries gets zero key
    gradients, one without keys empty rows."""
    torch = torch_cuda()
    fa = lib()
    log_case(test="packed-gaps", dtype=dtype)
    cfg = custom(5, d=64, dtype=dtype, H=2)
    total = 200
    t = {n: fi.make_head(cfg, n, 0, 0, 1, N=total * 2)[:total * 2].reshape(2, total, 64)
         for n in ("q", "k", "v", "do")}
    cu_q = np.array([3, 70, 70, 150], np.int32)       # rows 0..2 and 150.. belong to none
    cu_k = np.array([0, 90, 120, 120], np.int32)      # sequence 2 has no keys
    dev = {n: to_device(torch, t[n], dtype) for n in t}
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    sentinel = 3.0
    o = torch.full_like(dev["q"], sentinel)
    lse = torch.full((2, total), sentinel, dtype=torch.float32, device=o.device)
    fa.forward_varlen(dev["q"], dev["k"], dev["v"], cq, ck, 80, 90, scale=cfg.scale, causal=True,
                      out=o, lse=lse)
    grads = [torch.full_like(dev["q"], sentinel) for _ in range(3)]
    fa.backward_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cq, ck, 80, 90,
                       scale=cfg.scale, causal=True, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    outside_q = np.r_[0:3, 150:total]
    outside_k = np.r_[120:total]
    assert torch.all(o[:, outside_q] == sentinel) and torch.all(lse[:, outside_q] == sentinel)
    assert torch.all(grads[0][:, outside_q] == sentinel)
    assert torch.all(grads[1][:, outside_k] == sentinel)
    assert torch.all(grads[2][:, outside_k] == sentinel)
    # sequence 1 (queries 70..69: none) owns keys 90..119: zero gradients
    assert torch.count_nonzero(grads[1][:, 90:120]).item() == 0
    assert torch.count_nonzero(grads[2][:, 90:120]).item() == 0
    # sequence 2 (queries 70..149, no keys): empty rows, zero dq
    assert torch.count_nonzero(o[:, 70:150]).item() == 0
    assert torch.isneginf(lse[:, 70:150]).all().item()
    assert torch.count_nonzero(grads[0][:, 70:150]).item() == 0
    # the owned rows match the oracle
    w = {n: fi.widen(t[n], dtype) for n in t}
    ref_o, ref_l = oracle.attention_packed(w["q"], w["k"], w["v"], cu_q, cu_k, cfg.scale, True)
    got = from_device(o, dtype)
    assert max_abs(got[:, 3:150], ref_o[:, 3:150]) <= O_TOL[dtype]
    refs = oracle.attention_backward_packed(w["q"], w["k"], w["v"], ref_o, w["do"], ref_l, cu_q,
                                            cu_k, cfg.scale, True)
    for g, r, rows in zip(grads, refs, (np.r_[3:150], np.r_[0:120], np.r_[0:120])):
        gg = from_device(g, dtype)[:, rows]
        assert np.all(np.abs(gg - r[:, rows]) <= grad_bound(r[:, rows], dtype))
