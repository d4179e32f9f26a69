"""Python binding of the gfx950 exact-attention library (libfa_mi355x.so).

Two layers, both argument marshalling only (every step of the computation
runs in the HIP kernels behind the C ABI of include/fa.h):

* ``fa_forward``, ``fa_backward``, ``fa_backward_workspace_size``,
  ``fa_status_string``, ``fa_abi_version``: the C entry points under the same
  names, taking raw device addresses (ints) and returning status codes.
* ``forward`` / ``backward``: the same calls on torch tensors (PyTorch
  provides device memory and the current stream), raising ``FAError`` on any
  non-success status.

There is no fallback: if the shared library is missing, ``load_library``
raises ``FALibraryMissing``; build it with ``python -m exact_io_aware_41_amd.build``.
"""

from __future__ import annotations

import contextlib
import ctypes
import math
import os

__all__ = [
    "FA_SUCCESS", "FA_ERROR_INVALID_VALUE", "FA_ERROR_UNSUPPORTED", "FA_ERROR_LAUNCH",
    "FA_ERROR_SCRATCH_LIMIT", "FA_NOALLOC_SCRATCH_BYTES", "fa_backward_noalloc",
    "backward_noalloc",
    "FA_DTYPE_F32", "FA_DTYPE_BF16", "FA_DTYPE_F16", "EXPORTED_SYMBOLS",
    "FAError", "FALibraryMissing", "LIB_PATH", "DEBUG_LIB_PATH", "load_library",
    "load_debug_library", "library",
    "fa_abi_version", "fa_status_string", "fa_forward", "fa_backward",
    "fa_backward_workspace_size", "fa_backward_preprocess", "fa_backward_dkdv",
    "fa_backward_dq", "fa_forward_fp8", "fa_forward_varlen", "fa_backward_varlen", "fa_decode_workspace_size",
    "fa_decode", "fa_merge_states", "forward", "backward", "backward_phases", "forward_varlen",
    "backward_varlen", "forward_fp8", "decode", "merge_states",
]

FA_SUCCESS = 0
FA_ERROR_INVALID_VALUE = 1
FA_ERROR_UNSUPPORTED = 2
FA_ERROR_LAUNCH = 3
FA_ERROR_SCRATCH_LIMIT = 4
FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2

EXPORTED_SYMBOLS = ("fa_abi_version", "fa_status_string", "fa_forward",
                    "fa_backward_workspace_size", "fa_backward", "fa_backward_preprocess",
                    "fa_backward_dkdv", "fa_backward_dq", "fa_forward_fp8", "fa_forward_varlen",
                    "fa_backward_varlen", "fa_decode_workspace_size", "fa_decode",
                    "fa_merge_states", "fa_backward_noalloc")

# bytes of the static workspace fa_backward_noalloc uses on each GPU (one
# fp32 per query row of the batch)
FA_NOALLOC_SCRATCH_BYTES = 32 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_mi355x.so")
# the same library built with the race-check switches (NaN-poisoned LDS copy
# destinations, scrambled work-group order); for tests only
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_mi355x_debug.so")

_lib = None


class FAError(RuntimeError):
    """A non-success status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where} failed: {fa_status_string(status)} ({status})")


class FALibraryMissing(ImportError):
    pass


def load_library():
    """Load libfa_mi355x.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(LIB_PATH)
    return _lib


def load_debug_library():
    """The race-check build of the library (a separate handle; the torch
    wrappers use it inside ``with library(handle):``)."""
    return _open(DEBUG_LIB_PATH)


@contextlib.contextmanager
def library(handle):
    """Route every call of this module to `handle` inside the block."""
    global _lib
    old = load_library()
    _lib = handle
    try:
        yield handle
    finally:
        _lib = old


def _open(path):
    if not os.path.exists(path):
        raise FALibraryMissing(
            f"{path} is not built; run `python -m exact_io_aware_41_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_abi_version.restype = i32
    lib.fa_abi_version.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i32]
    lib.fa_forward.restype = i32
    lib.fa_forward.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, f32, i32, vp, vp,
                               vp]
    lib.fa_backward_workspace_size.restype = sz
    lib.fa_backward_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_backward.restype = i32
    lib.fa_backward.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32,
                                i32, vp, vp, vp, vp, sz, vp]
    lib.fa_backward_noalloc.restype = i32
    lib.fa_backward_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                        f32, i32, vp, vp, vp, vp]
    lib.fa_backward_preprocess.restype = i32
    lib.fa_backward_preprocess.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.fa_backward_dkdv.restype = i32
    lib.fa_backward_dkdv.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                     f32, i32, vp, vp, vp]
    lib.fa_backward_dq.restype = i32
    lib.fa_backward_dq.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32,
                                   i32, vp, vp]
    lib.fa_forward_fp8.restype = i32
    lib.fa_forward_fp8.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, f32, f32, f32, f32,
                                   i32, vp, vp, vp]
    lib.fa_forward_varlen.restype = i32
    lib.fa_forward_varlen.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                      f32, i32, vp, vp, vp]
    lib.fa_backward_varlen.restype = i32
    lib.fa_backward_varlen.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                       vp, vp, vp, f32, i32, vp, vp, vp, vp, sz, vp]
    lib.fa_decode_workspace_size.restype = sz
    lib.fa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_decode.restype = i32
    lib.fa_decode.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.fa_merge_states.restype = i32
    lib.fa_merge_states.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    return lib


# ---------------------------------------------------------------------------
# C entry points (raw addresses)
# ---------------------------------------------------------------------------

def fa_abi_version() -> int:
    return load_library().fa_abi_version()


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_forward(dtype, B, H, Nq, Nk, d, q, k, v, seqlens_k, scale, causal, o, lse,
               stream=0) -> int:
    return load_library().fa_forward(dtype, B, H, Nq, Nk, d, q, k, v, seqlens_k, scale, causal,
                                     o, lse, stream)


def fa_backward_workspace_size(dtype, B, H, N, d) -> int:
    return load_library().fa_backward_workspace_size(dtype, B, H, N, d)


def fa_backward(dtype, B, H, Nq, Nk, d, q, k, v, o, dout, lse, seqlens_k, scale, causal, dq, dk,
                dv, workspace, workspace_bytes, stream=0) -> int:
    return load_library().fa_backward(dtype, B, H, Nq, Nk, d, q, k, v, o, dout, lse, seqlens_k,
                                      scale, causal, dq, dk, dv, workspace, workspace_bytes,
                                      stream)


def fa_backward_noalloc(dtype, B, H, Nq, Nk, d, q, k, v, o, dout, lse, seqlens_k, scale, causal,
                        dq, dk, dv, stream=0) -> int:
    return load_library().fa_backward_noalloc(dtype, B, H, Nq, Nk, d, q, k, v, o, dout, lse,
                                              seqlens_k, scale, causal, dq, dk, dv, stream)


def fa_backward_preprocess(dtype, B, H, N, d, o, dout, delta, stream=0) -> int:
    return load_library().fa_backward_preprocess(dtype, B, H, N, d, o, dout, delta, stream)


def fa_backward_dkdv(dtype, B, H, Nq, Nk, d, q, k, v, dout, lse, delta, seqlens_k, scale, causal,
                     dk, dv, stream=0) -> int:
    return load_library().fa_backward_dkdv(dtype, B, H, Nq, Nk, d, q, k, v, dout, lse, delta,
                                           seqlens_k, scale, causal, dk, dv, stream)


def fa_backward_dq(dtype, B, H, Nq, Nk, d, q, k, v, dout, lse, delta, seqlens_k, scale, causal,
                   dq, stream=0) -> int:
    return load_library().fa_backward_dq(dtype, B, H, Nq, Nk, d, q, k, v, dout, lse, delta,
                                         seqlens_k, scale, causal, dq, stream)


def fa_forward_fp8(B, H, Nq, Nk, d, q, k, v, seqlens_k, scale, q_descale, k_descale, v_descale,
                   causal, o, lse, stream=0) -> int:
    return load_library().fa_forward_fp8(B, H, Nq, Nk, d, q, k, v, seqlens_k, scale, q_descale,
                                         k_descale, v_descale, causal, o, lse, stream)


def fa_forward_varlen(dtype, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k, d, q, k, v,
                      cu_seqlens_q, cu_seqlens_k, scale, causal, o, lse, stream=0) -> int:
    return load_library().fa_forward_varlen(dtype, B, H, total_q, total_k, max_seqlen_q,
                                            max_seqlen_k, d, q, k, v, cu_seqlens_q, cu_seqlens_k,
                                            scale, causal, o, lse, stream)


def fa_backward_varlen(dtype, B, H, total_q, total_k, max_seqlen_q, max_seqlen_k, d, q, k, v, o,
                       dout, lse, cu_seqlens_q, cu_seqlens_k, scale, causal, dq, dk, dv,
                       workspace, workspace_bytes, stream=0) -> int:
    return load_library().fa_backward_varlen(dtype, B, H, total_q, total_k, max_seqlen_q,
                                             max_seqlen_k, d, q, k, v, o, dout, lse,
                                             cu_seqlens_q, cu_seqlens_k, scale, causal, dq, dk,
                                             dv, workspace, workspace_bytes, stream)


def fa_decode_workspace_size(dtype, B, H, N, d) -> int:
    return load_library().fa_decode_workspace_size(dtype, B, H, N, d)


def fa_decode(dtype, B, H, N, d, q, k, v, seqlens_k, scale, o, lse, workspace, workspace_bytes,
              stream=0) -> int:
    return load_library().fa_decode(dtype, B, H, N, d, q, k, v, seqlens_k, scale, o, lse,
                                    workspace, workspace_bytes, stream)


def fa_merge_states(dtype, rows, n_parts, d, o_parts, lse_parts, o, lse, stream=0) -> int:
    return load_library().fa_merge_states(dtype, rows, n_parts, d, o_parts, lse_parts, o, lse,
                                          stream)


# ---------------------------------------------------------------------------
# torch tensor wrappers
# ---------------------------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise FAError(FA_ERROR_UNSUPPORTED, f"dtype {t.dtype}")


def _check_like(name, t, ref):
    if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
        raise ValueError(f"{name} must match q in shape, dtype and device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_keys(name, t, k, q):
    """k-shaped tensors: [B, H, Nk, d] with q's batch, heads, head dim, dtype
    and device."""
    if (t.dim() != 4 or t.shape != k.shape or t.shape[0] != q.shape[0]
            or t.shape[1] != q.shape[1] or t.shape[3] != q.shape[3]
            or t.dtype != q.dtype or t.device != q.device):
        raise ValueError(f"{name} must be [B, H, Nk, d] like k, with q's B, H, d, dtype and "
                         f"device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_q_k(q, k):
    """q [B, H, Nq, d] and k [B, H, Nk, d], q dense: the kernels index q as a
    contiguous row-major tensor, so a strided view must be rejected here."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k [B, H, Nk, d]")
    _check_like("q", q, q)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _lengths(seqlens_k, q):
    import torch
    if seqlens_k is None:
        return None
    if (seqlens_k.dtype != torch.int32 or seqlens_k.device != q.device
            or seqlens_k.shape != (q.shape[0],) or not seqlens_k.is_contiguous()):
        raise ValueError("seqlens_k must be a contiguous int32 [B] tensor on q's device")
    return seqlens_k


def forward(q, k, v, scale=None, causal=False, seqlens_k=None, out=None, lse=None):
    """O, LSE = attention(q, k, v) for CUDA tensors q [B, H, Nq, d] and
    k, v [B, H, Nk, d] (usually Nq == Nk).

    ``scale`` defaults to 1/sqrt(d); ``seqlens_k`` is an optional int32 [B]
    tensor of key lengths; with ``causal`` query i sees keys j <= i + Nk - Nq.
    Returns (o, lse) with o like q and lse fp32 [B, H, Nq].
    """
    import torch
    _check_q_k(q, k)
    for name, t in (("k", k), ("v", v)):
        _check_keys(name, t, k, q)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqlens_k = _lengths(seqlens_k, q)
    if out is None:
        out = torch.empty_like(q)
    _check_like("out", out, q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    st = fa_forward(_dtype_code(q), B, H, N, Nk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens_k),
                    float(scale), int(bool(causal)), _ptr(out), _ptr(lse), _stream(q.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_forward")
    return out, lse


def backward(q, k, v, o, do, lse, scale=None, causal=False, seqlens_k=None,
             dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of <dO, O> for the tensors of a previous ``forward`` call
    (q, o, do, dq [B, H, Nq, d]; k, v, dk, dv [B, H, Nk, d])."""
    import torch
    _check_q_k(q, k)
    for name, t in (("o", o), ("do", do)):
        _check_like(name, t, q)
    for name, t in (("k", k), ("v", v)):
        _check_keys(name, t, k, q)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqlens_k = _lengths(seqlens_k, q)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check_like("dq", dq, q)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_keys(name, t, k, q)
    code = _dtype_code(q)
    ws_bytes = fa_backward_workspace_size(code, B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    st = fa_backward(code, B, H, N, Nk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                     _ptr(seqlens_k), float(scale), int(bool(causal)), _ptr(dq), _ptr(dk),
                     _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                     _stream(q.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_backward")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False,
                     seqlens_k=None):
    """``backward`` through fa_backward_noalloc: the caller supplies every
    output, nothing is allocated (the workspace is the library's static
    per-GPU array); returns (dq, dk, dv)."""
    import torch
    _check_q_k(q, k)
    for name, t in (("o", o), ("do", do), ("dq", dq)):
        _check_like(name, t, q)
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _check_keys(name, t, k, q)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqlens_k = _lengths(seqlens_k, q)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    st = fa_backward_noalloc(_dtype_code(q), B, H, N, Nk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                             _ptr(do), _ptr(lse), _ptr(seqlens_k), float(scale),
                             int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _stream(q.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_backward_noalloc")
    return dq, dk, dv


def forward_fp8(q, k, v, q_descale, k_descale, v_descale, scale=None, causal=False,
                seqlens_k=None, out=None, lse=None):
    """Attention of FP8 inputs: q [B, H, Nq, d], k, v [B, H, Nk, d] hold OCP
    E4M3 codes (torch.float8_e4m3fn, or uint8 bytes), the real values being
    code * descale.  Returns (o bf16 like q, lse fp32 [B, H, Nq])."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[:2] != q.shape[:2] \
            or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8) or t.device != q.device \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous E4M3 codes on q's device")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqlens_k = _lengths(seqlens_k, q)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    st = fa_forward_fp8(B, H, N, Nk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens_k), float(scale),
                        float(q_descale), float(k_descale), float(v_descale), int(bool(causal)),
                        _ptr(out), _ptr(lse), _stream(q.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_forward_fp8")
    return out, lse


def _check_packed(q, k, v, cu_seqlens_q, cu_seqlens_k):
    """q [H, total_q, d]; k, v [H, total_k, d] with q's H, d, dtype, device;
    int32 [B + 1] offsets on q's device.  Returns B."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[0] != q.shape[0] \
            or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [H, total_q, d] and k, v [H, total_k, d]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with q's dtype and device")
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if (cu.dtype != torch.int32 or cu.device != q.device or cu.dim() != 1
                or cu.numel() < 1 or not cu.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 [B + 1] tensor on q's device")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    return cu_seqlens_q.numel() - 1


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                   causal=False, out=None, lse=None):
    """Attention over a packed batch: sequence b owns query rows
    cu_seqlens_q[b]:cu_seqlens_q[b+1] of q [H, total_q, d] and key rows
    cu_seqlens_k[b]:cu_seqlens_k[b+1] of k, v [H, total_k, d]; each sequence
    is its own problem (causal: query i of the sequence sees its keys
    j <= i + nk_b - nq_b).  ``max_seqlen_q`` / ``max_seqlen_k`` bound every
    sequence's lengths.  Returns (o like q, lse fp32 [H, total_q]); rows of
    no sequence are o = 0, lse = -inf when the outputs are allocated here.
    """
    import torch
    B = _check_packed(q, k, v, cu_seqlens_q, cu_seqlens_k)
    H, total_q, d = q.shape
    total_k = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.zeros_like(q)
    _check_like("out", out, q)
    if lse is None:
        lse = torch.full((H, total_q), -math.inf, dtype=torch.float32, device=q.device)
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [H, total_q] tensor")
    st = fa_forward_varlen(_dtype_code(q), B, H, total_q, total_k, int(max_seqlen_q),
                           int(max_seqlen_k), d, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                           _ptr(cu_seqlens_k), float(scale), int(bool(causal)), _ptr(out),
                           _ptr(lse), _stream(q.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_forward_varlen")
    return out, lse


def backward_varlen(q, k, v, o, do, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of <dO, O> for a previous ``forward_varlen`` call, in the
    packed layout; rows of no sequence are zero when the outputs are
    allocated here."""
    import torch
    B = _check_packed(q, k, v, cu_seqlens_q, cu_seqlens_k)
    for name, t in (("o", o), ("do", do)):
        _check_like(name, t, q)
    H, total_q, d = q.shape
    total_k = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [H, total_q] tensor")
    dq = torch.zeros_like(q) if dq is None else dq
    dk = torch.zeros_like(k) if dk is None else dk
    dv = torch.zeros_like(k) if dv is None else dv
    _check_like("dq", dq, q)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_like(name, t, k)
    code = _dtype_code(q)
    ws_bytes = fa_backward_workspace_size(code, 1, H, total_q, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    st = fa_backward_varlen(code, B, H, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), d,
                            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                            _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), float(scale),
                            int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_backward_varlen")
    return dq, dk, dv


def backward_phases(q, k, v, o, do, lse, scale=None, causal=False, seqlens_k=None,
                    dq=None, dk=None, dv=None, delta=None, events=None):
    """``backward`` issued as its three launches (preprocess, dK/dV, dQ).

    If ``events`` is a list of four torch.cuda.Event objects they are recorded
    on the current stream before, between and after the launches, so each
    launch can be timed on the stream it runs on.
    """
    import torch
    _check_q_k(q, k)
    for name, t in (("o", o), ("do", do)):
        _check_like(name, t, q)
    for name, t in (("k", k), ("v", v)):
        _check_keys(name, t, k, q)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqlens_k = _lengths(seqlens_k, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check_like("dq", dq, q)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_keys(name, t, k, q)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if (delta.shape != (B, H, N) or delta.dtype != torch.float32 or delta.device != q.device
            or not delta.is_contiguous()):
        raise ValueError("delta must be a contiguous fp32 [B, H, N] tensor on q's device")
    code = _dtype_code(q)
    stream = _stream(q.device)
    rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)
    rec(0)
    st = fa_backward_preprocess(code, B, H, N, d, _ptr(o), _ptr(do), _ptr(delta), stream)
    if st != FA_SUCCESS:
        raise FAError(st, "fa_backward_preprocess")
    rec(1)
    st = fa_backward_dkdv(code, B, H, N, Nk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
                          _ptr(delta), _ptr(seqlens_k), float(scale), int(bool(causal)), _ptr(dk),
                          _ptr(dv), stream)
    if st != FA_SUCCESS:
        raise FAError(st, "fa_backward_dkdv")
    rec(2)
    st = fa_backward_dq(code, B, H, N, Nk, d, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
                        _ptr(delta), _ptr(seqlens_k), float(scale), int(bool(causal)), _ptr(dq),
                        stream)
    if st != FA_SUCCESS:
        raise FAError(st, "fa_backward_dq")
    rec(3)
    return dq, dk, dv


def decode(q, k, v, scale=None, seqlens_k=None, out=None, lse=None, workspace=None):
    """O, LSE of one query row per (batch, head) against a key/value cache.

    q: [B, H, d]; k, v: [B, H, N, d] (cache of capacity N); ``seqlens_k`` an
    optional int32 [B] tensor of cached lengths.  Returns (o [B, H, d] in q's
    dtype, lse fp32 [B, H]).
    """
    import torch
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, H, d] and k, v [B, H, N, d]")
    B, H, N, d = k.shape
    if q.shape != (B, H, d) or q.dtype != k.dtype or q.device != k.device or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, H, d] tensor like k")
    _check_like("v", v, k)
    if not k.is_contiguous():
        raise ValueError("k must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqlens_k = _lengths(seqlens_k, k)
    out = torch.empty_like(q) if out is None else out
    _check_like("out", out, q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if lse.shape != (B, H) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H] tensor")
    code = _dtype_code(q)
    ws_bytes = fa_decode_workspace_size(code, B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    st = fa_decode(code, B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens_k), float(scale),
                   _ptr(out), _ptr(lse), _ptr(workspace),
                   workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_decode")
    return out, lse


def merge_states(o_parts, lse_parts, dtype=None, out=None, lse=None):
    """Merge partial results over disjoint key sets.

    o_parts: fp32 [R, S, d]; lse_parts: fp32 [R, S].  Returns (o [R, d] in
    ``dtype`` (default fp32), lse fp32 [R]).
    """
    import torch
    if o_parts.dim() != 3 or o_parts.dtype != torch.float32 or not o_parts.is_contiguous():
        raise ValueError("o_parts must be a contiguous fp32 [R, S, d] tensor")
    R, S, d = o_parts.shape
    if (lse_parts.shape != (R, S) or lse_parts.dtype != torch.float32
            or not lse_parts.is_contiguous() or lse_parts.device != o_parts.device):
        raise ValueError("lse_parts must be a contiguous fp32 [R, S] tensor on o_parts' device")
    dtype = torch.float32 if dtype is None else dtype
    out = torch.empty((R, d), dtype=dtype, device=o_parts.device) if out is None else out
    if out.shape != (R, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [R, d] tensor")
    if lse is None:
        lse = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
    st = fa_merge_states(_dtype_code(out), R, S, d, _ptr(o_parts), _ptr(lse_parts), _ptr(out),
                         _ptr(lse), _stream(o_parts.device))
    if st != FA_SUCCESS:
        raise FAError(st, "fa_merge_states")
    return out, lse
