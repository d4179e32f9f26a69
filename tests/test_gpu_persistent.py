"""Parity on the GPU for the persistent forward launch.

A padded problem (no key lengths) with more query tiles than the chip holds
work-groups at once runs one work-group per slot, each working through a
fixed list of query tiles ("FlashAttention", "Checking it on a real system":
the kernel's schedule must not change what it computes).  For every head
dimension and both masks, at 20 heads and 8192 rows (640 to 1280 query tiles):

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
N = 8192


@pytest.mark.parametrize("dtype, d, causal, H", [
    ("bf16", 64, True, 20), ("bf16", 64, False, 24),
    ("bf16", 96, True, 20),
    ("bf16", 128, True, 20), ("bf16", 128, False, 20), ("f16", 128, True, 24),
    ("bf16", 192, True, 20),
    ("bf16", 256, True, 20), ("bf16", 256, False, 16),
])
def test_persistent_forward_matches_per_tile_launch_and_oracle(dtype, d, causal, H):
    torch = torch_cuda()
    fa = lib()
    log_case(test="persistent-forward", dtype=dtype, d=d, causal=causal, H=H, N=N)
    cfg = custom(3, d=d, dtype=dtype, H=H, N=N)
    t = {n: fi.make_tensor(cfg, n, seed=11, d=d) for n in ("q", "k", "v")}
    dev = {n: to_device(torch, t[n], dtype) for n in t}
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=causal)

    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda")
    o_p, lse_p = fa.forward_varlen(dev["q"][0], dev["k"][0], dev["v"][0], cu, cu, N, N,
                                   scale=cfg.scale, causal=causal)
    with fa.library(fa.load_debug_library()):
        o_d, lse_d = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o[0], o_p), "O differs from the one-work-group-per-tile launch"
    assert torch.equal(lse[0], lse_p), "LSE differs from the one-work-group-per-tile launch"
    assert not o_d.float().isnan().any().item(), "NaN under the race-check library"
    assert torch.equal(o, o_d), "O differs under the race-check library"
    assert torch.equal(lse, lse_d), "LSE differs under the race-check library"

    got_o, got_l = from_device(o[0], dtype), lse[0].cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(d + 7 * H)
    edges = np.arange(0, N, 128)
    rows = np.unique(np.concatenate([edges, edges + 127, rng.integers(0, N, 8)]))
    for h in (0, int(rng.integers(1, H - 1)), H - 1):
        q = fi.widen(t["q"][0, h], dtype)
        k = fi.widen(t["k"][0, h], dtype)
        v = fi.widen(t["v"][0, h], dtype)
        ref_o, ref_l = oracle.attention_rows(q, k, v, rows, cfg.scale, causal)
        err = max_abs(got_o[h, rows], ref_o)
        print(f"head {h}: max |O - ref| = {err:.3e} over {len(rows)} rows", flush=True)
        assert err <= O_TOL[dtype]
        check_lse(got_l[h, rows], ref_l, *LSE_TOL[dtype])
