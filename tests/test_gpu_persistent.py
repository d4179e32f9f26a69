"""Parity on the GPU for the persistent forward launch.

A padded problem (no key lengths) with more query tiles than the chip holds
work-groups at once runs one work-group per slot, each working through a
fixed list of query tiles ("FlashAttention", "Checking it on a real system":
the kernel's schedule must not change what it computes).  For every head
dimension and both masks, at 16 to 24 heads and 8192 rows (512 to 1536 query
tiles), and for ragged lengths, two sequences, and fewer or more keys than
queries (so that some jobs see no key at all):

* bit for bit against the same problem given as a packed batch of one
  sequence, which keeps one work-group per query tile, and against the
  race-check library (every copy destination filled with NaN before the copy,
  jobs taken in a scrambled order), where a job that read a ring slot the
  previous or next job of its work-group still used would show;
* the first and last row of every 128-row block and a few random rows of
  three heads against the fp64 oracle, one row at a time (O <= 2e-2 for bf16,
  5e-3 for f16; LSE within the forward tolerances).
"""

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import (LSE_TOL, check_lse, custom, from_device, lib, log_case, max_abs,
                               to_device, torch_cuda)

pytestmark = pytest.mark.gpu

O_TOL = {"bf16": 2e-2, "f16": 5e-3}


def _check(dtype, d, causal, B, H, Nq, Nk, seed=11):
    torch = torch_cuda()
    fa = lib()
    log_case(test="persistent-forward", dtype=dtype, d=d, causal=causal, B=B, H=H, Nq=Nq, Nk=Nk)
    cfg = custom(3, d=d, dtype=dtype, B=B, H=H, N=Nq)
    t = {"q": fi.make_tensor(cfg, "q", seed=seed, d=d, N=Nq)}
    t.update({n: fi.make_tensor(cfg, n, seed=seed, d=d, N=Nk) for n in ("k", "v")})
    dev = {n: to_device(torch, t[n], dtype) for n in t}
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=causal)

    # the same problem as a packed batch: one work-group per query tile
    packed = {n: dev[n].permute(1, 0, 2, 3).reshape(H, -1, d).contiguous() for n in dev}
    cu_q = torch.arange(0, B + 1, dtype=torch.int32, device="cuda") * Nq
    cu_k = torch.arange(0, B + 1, dtype=torch.int32, device="cuda") * Nk
    o_p, lse_p = fa.forward_varlen(packed["q"], packed["k"], packed["v"], cu_q, cu_k, Nq, Nk,
                                   scale=cfg.scale, causal=causal)
    with fa.library(fa.load_debug_library()):
        o_d, lse_d = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=causal)
    torch.cuda.synchronize()
    o_pb = o_p.reshape(H, B, Nq, d).permute(1, 0, 2, 3)
    lse_pb = lse_p.reshape(H, B, Nq).permute(1, 0, 2)
    assert torch.equal(o, o_pb), "O differs from the one-work-group-per-tile launch"
    assert torch.equal(lse, lse_pb), "LSE differs from the one-work-group-per-tile launch"
    assert not o_d.float().isnan().any().item(), "NaN under the race-check library"
    assert torch.equal(o, o_d), "O differs under the race-check library"
    assert torch.equal(lse, lse_d), "LSE differs under the race-check library"

    got_o, got_l = from_device(o, dtype), lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(d + 7 * H + Nq + 3 * Nk)
    edges = np.arange(0, Nq, 128)
    rows = np.unique(np.concatenate([edges, np.minimum(edges + 127, Nq - 1), [Nq - 1],
                                     rng.integers(0, Nq, 8)]))
    for b, h in ((0, 0), (B - 1, int(rng.integers(1, H - 1))), (B - 1, H - 1)):
        q = fi.widen(t["q"][b, h], dtype)
        k = fi.widen(t["k"][b, h], dtype)
        v = fi.widen(t["v"][b, h], dtype)
        ref_o, ref_l = oracle.attention_rows(q, k, v, rows, cfg.scale, causal)
        err = max_abs(got_o[b, h, rows], ref_o)
        print(f"(b, h) = ({b}, {h}): max |O - ref| = {err:.3e} over {len(rows)} rows", flush=True)
        assert err <= O_TOL[dtype]
        check_lse(got_l[b, h, rows], ref_l, *LSE_TOL[dtype])
        assert np.all(got_o[b, h, rows][np.isneginf(ref_l)] == 0.0)


@pytest.mark.parametrize("dtype, d, causal, H", [
    ("bf16", 64, True, 20), ("bf16", 64, False, 24),
    ("bf16", 96, True, 20),
    ("bf16", 128, True, 20), ("bf16", 128, False, 20), ("f16", 128, True, 24),
    ("bf16", 192, True, 20),
    ("bf16", 256, True, 20), ("bf16", 256, False, 16),
])
def test_persistent_forward_matches_per_tile_launch_and_oracle(dtype, d, causal, H):
    _check(dtype, d, causal, 1, H, 8192, 8192)


@pytest.mark.parametrize("d, causal, B, H, Nq, Nk", [
    (128, True, 2, 12, 8000, 8000),    # ragged last query tile, two sequences (24 heads)
    (128, True, 1, 20, 8192, 4096),    # fewer keys: the first 4096 queries see none
    (128, True, 1, 20, 4096, 8192),    # more keys than queries
    (96, False, 1, 20, 6000, 3000),
    (256, True, 1, 16, 5000, 6000),
])
def test_persistent_forward_ragged_and_rectangular(d, causal, B, H, Nq, Nk):
    _check("bf16", d, causal, B, H, Nq, Nk, seed=13)
