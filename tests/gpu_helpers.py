"""Shared plumbing for the GPU parity tests: device upload of the seeded
inputs, calls through the binding, and exact widening of the results.

On a machine with a GPU the HIP library must be present: a missing library
is a failure, never a skip or a fallback.
"""

from __future__ import annotations

import dataclasses

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
