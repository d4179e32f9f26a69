"""Shared plumbing for the GPU parity tests: device upload of the seeded
inputs, calls through the binding, and exact widening of the results.

On a machine with a GPU the HIP library must be present: a missing library
is a failure, never a skip or a fallback.
"""

from __future__ import annotations

import dataclasses
import math
import os

import numpy as np
import pytest

import fa_inputs as fi


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def lib():
    import exact_io_aware_41_amd as fa
    fa.load_library()          # raises FALibraryMissing: never skipped on a GPU machine
    return fa


def log_case(**kw):
    print("CASE " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def custom(cfg_id=2, **kw):
    """A workload derived from one of the five, with fields overridden."""
    return dataclasses.replace(fi.CONFIGS[cfg_id], **kw)


def torch_dtype(torch, dtype):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


def to_device(torch, arr, dtype):
    if dtype in fi.HALF_DTYPES:
        bits = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda()
        return bits.view(torch_dtype(torch, dtype))
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def from_device(t, dtype):
    """Exact float64 values of a device tensor (bf16, f16 or fp32)."""
    import torch
    if dtype in fi.HALF_DTYPES:
        bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return fi.widen(bits, dtype)
    return t.detach().cpu().numpy().astype(np.float64)


def device_inputs(torch, cfg, inputs):
    dev = {n: to_device(torch, inputs[n], cfg.dtype) for n in ("q", "k", "v", "do") if n in inputs}
    lens = inputs.get("lengths")
    dev["lengths"] = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    return dev


def max_abs(a, b):
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def check_lse(gpu, ref, tol_abs, tol_rel=0.0):
    """-inf must match exactly; finite entries within tol_abs + tol_rel*|ref|."""
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu), ninf), "empty-row LSE must be exactly -inf"
    assert not np.any(np.isnan(gpu))
    fin = ~ninf
    err = np.abs(gpu[fin] - ref[fin])
    bound = tol_abs + tol_rel * np.abs(ref[fin])
    assert np.all(err <= bound), f"LSE error {err.max() if err.size else 0:.3e}"
    return float(err.max()) if err.size else 0.0


# LSE tolerance (abs, rel) of the forward per element format.  In the 16-bit
# kernels the running sum l adds the weights after their rounding to the MFMA
# operand format (the weights O is built from), each within a relative
# u = 2^-8 (bf16) or 2^-11 (f16) of its exact value, so ln l may differ from
# the exact log-sum-exp by up to ln(1 + u): 3.9e-3 for bf16; f16's 4.9e-4 fits
# the 1e-3 it has always been held to.  Plus 1e-4 for fp32 accumulation and
# 1e-5 |LSE| for the fp32 result at large magnitudes.  fp32 inputs: fp32
# weights throughout.
LSE_TOL = {"f32": (1e-5, 0.0), "bf16": (math.log1p(2.0 ** -8) + 1e-4, 1e-5), "f16": (1e-3, 1e-5)}

# Gradient tolerances (dQ, dK, dV max abs) per element format, and the
# relative size of one unit in the last place of that format.
G_TOL = {"bf16": 5e-2, "f16": 2e-2, "f32": 1e-4}
ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -20}
PRECISION_BITS = {"bf16": 8, "f16": 11, "f32": 24}


def half_ulp_threshold(dtype, tol):
    """Smallest magnitude 2^e at which half an ulp of the format, 2^(e - p)
    for p significand bits, exceeds `tol`: below it one rounding of the
    output fits inside the tolerance (bf16 at 5e-2: 16; f16 at 2e-2: 64;
    fp32 at 1e-4: 2048)."""
    p = PRECISION_BITS[dtype]
    return 2.0 ** (math.floor(math.log2(tol)) + 1 + p)


def grad_bound(ref, dtype):
    """Per-element bound on |gpu - ref| for a gradient: the format's stated
    tolerance, plus one ulp of |ref| only where |ref| reaches the magnitude at
    which a half-ulp of the output format alone exceeds that tolerance."""
    tol = G_TOL[dtype]
    a = np.abs(ref)
    return tol + np.where(a >= half_ulp_threshold(dtype, tol), ULP[dtype] * a, 0.0)


def host_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def parallel_map(fn, items):
    """fn over items on a thread pool sized to this host's cores, BLAS held
    to one thread per worker (the oracle's NumPy kernels release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    items = list(items)
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(host_workers()) as ex:
            return list(ex.map(fn, items))


def oracle_head_rows(oracle, q, k, v, scale, causal, length=None, rows=None, chunk=256):
    """Route A on the given rows (all rows by default) of one head, the rows
    cut into chunks computed in parallel.  Returns (o, lse) in row order."""
    N = q.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    parts = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    res = parallel_map(lambda r: oracle.attention_rows(q, k, v, r, scale, causal, length), parts)
    if not res:
        return np.zeros((0, v.shape[1])), np.zeros(0)
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
