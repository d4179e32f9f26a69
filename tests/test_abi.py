"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/fa.h declares, and rejects invalid calls before any HIP call."""

import ctypes
import math
import os
import re
import subprocess

import pytest

import exact_io_aware_41_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.LIB_PATH),
                                reason="library not built (run __graft_entry__.build())")

BF16, F32, F16 = fa.FA_DTYPE_BF16, fa.FA_DTYPE_F32, fa.FA_DTYPE_F16
A = 0x10000          # aligned fake address: never dereferenced by these calls
MIS = 0x10004        # 4-byte aligned, not 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert names == sorted(fa.EXPORTED_SYMBOLS)
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert set(names) <= exported


def test_race_check_library_exports_the_same_calls():
    """The race-check build (NaN-poisoned copy destinations, scrambled
    work-group order) is the same C ABI, so the binding can drive it."""
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", fa.DEBUG_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert set(names) <= set(re.findall(r"\bT (fa_\w+)", out))
    dbg = fa.load_debug_library()
    assert dbg.fa_abi_version() == fa.fa_abi_version()
    with fa.library(dbg):
        assert fa.fa_abi_version() == 5
        assert fa.load_library() is dbg
    assert fa.load_library() is not dbg


def test_version_and_status_strings():
    assert fa.fa_abi_version() == 5
    assert fa.fa_status_string(fa.FA_SUCCESS) == "FA_SUCCESS"
    assert fa.fa_status_string(fa.FA_ERROR_INVALID_VALUE) == "FA_ERROR_INVALID_VALUE"
    assert fa.fa_status_string(fa.FA_ERROR_UNSUPPORTED) == "FA_ERROR_UNSUPPORTED"
    assert fa.fa_status_string(fa.FA_ERROR_LAUNCH) == "FA_ERROR_LAUNCH"
    assert fa.fa_status_string(fa.FA_ERROR_SCRATCH_LIMIT) == "FA_ERROR_SCRATCH_LIMIT"
    assert fa.fa_status_string(99) == "FA_ERROR_UNKNOWN"


def test_library_imports_no_allocation_routine():
    """No entry point can allocate device or host memory: the library does
    not even import the HIP allocation routines."""
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    alloc = {n for n in names if re.match(r"hip(Ext)?(Host)?(Malloc|Free|MemAlloc|HostAlloc|"
                                          r"MallocManaged|MallocAsync|FreeAsync|HostRegister)", n)}
    assert not alloc, alloc
    assert "hipGetSymbolAddress" in names


def noalloc(dtype=BF16, B=1, H=1, N=16, d=128, Nk=None, scale=0.1, causal=0, p=A):
    Nk = N if Nk is None else Nk
    return fa.fa_backward_noalloc(dtype, B, H, N, Nk, d, p, p, p, p, p, p, None, scale, causal,
                                  p, p, p, None)


def test_backward_noalloc_limits_without_a_gpu():
    """Checks that run before any HIP call: a problem whose row statistics
    exceed the static workspace is refused, an empty one succeeds."""
    rows = fa.FA_NOALLOC_SCRATCH_BYTES // 4
    assert rows == 8 * 32 * 32768
    assert noalloc(B=1, H=1, N=rows + 1) == fa.FA_ERROR_SCRATCH_LIMIT
    assert noalloc(B=8, H=32, N=32768 + 1) == fa.FA_ERROR_SCRATCH_LIMIT
    assert noalloc(B=0) == fa.FA_SUCCESS
    assert noalloc(H=0) == fa.FA_SUCCESS
    assert noalloc(N=0, Nk=0) == fa.FA_SUCCESS


def fwd(dtype=BF16, B=1, H=1, N=16, d=128, q=A, k=A, v=A, lens=None, scale=0.1, causal=0, o=A,
        lse=A, Nk=None):
    Nk = N if Nk is None else Nk
    return fa.fa_forward(dtype, B, H, N, Nk, d, q, k, v, lens, scale, causal, o, lse, None)


def bwd(dtype=BF16, B=1, H=1, N=16, d=128, scale=0.1, causal=0, ws=A, ws_bytes=1 << 20,
        Nk=None, **ptrs):
    Nk = N if Nk is None else Nk
    p = dict(q=A, k=A, v=A, o=A, do=A, lse=A, lens=None, dq=A, dk=A, dv=A)
    p.update(ptrs)
    return fa.fa_backward(dtype, B, H, N, Nk, d, p["q"], p["k"], p["v"], p["o"], p["do"],
                          p["lse"], p["lens"], scale, causal, p["dq"], p["dk"], p["dv"], ws,
                          ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(dtype=7), dict(B=-1), dict(H=-2), dict(N=-1), dict(d=0), dict(d=-128),
    dict(scale=0.0), dict(scale=-0.5), dict(scale=math.nan), dict(scale=math.inf),
    dict(causal=2), dict(causal=-1),
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(q=MIS), dict(k=MIS), dict(v=MIS), dict(o=MIS), dict(lse=MIS), dict(lens=A + 2),
])
def test_forward_rejects_invalid_arguments(kw):
    assert fwd(**kw) == fa.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("dtype,d", [(BF16, 80), (BF16, 512), (BF16, 32), (F32, 160), (F32, 16),
                                     (F32, 224), (F16, 160), (F16, 512), (BF16, 100)])
def test_forward_unsupported_shapes_fail_loudly(dtype, d):
    assert fwd(dtype=dtype, d=d) == fa.FA_ERROR_UNSUPPORTED


def test_forward_empty_problems_succeed_without_pointers():
    for B, H, N in ((0, 4, 16), (2, 0, 16), (2, 4, 0)):
        assert fwd(B=B, H=H, N=N, q=None, k=None, v=None, o=None, lse=None) == fa.FA_SUCCESS
    # an empty problem with an unsupported head dim still reports it
    assert fwd(N=0, d=160) == fa.FA_ERROR_UNSUPPORTED
    # f16 is a known format; an unknown code is an invalid value
    assert fwd(dtype=F16, N=0, q=None, k=None, v=None, o=None, lse=None) == fa.FA_SUCCESS
    assert fwd(dtype=3) == fa.FA_ERROR_INVALID_VALUE


def test_rectangular_problems_validate():
    assert fwd(Nk=-1) == fa.FA_ERROR_INVALID_VALUE
    # no query rows: nothing to write, pointers may be absent
    assert fwd(N=0, Nk=32, q=None, k=None, v=None, o=None, lse=None) == fa.FA_SUCCESS
    # queries without keys still write empty rows, so they need their buffers
    assert fwd(N=8, Nk=0, q=None) == fa.FA_ERROR_INVALID_VALUE
    assert bwd(Nk=-3) == fa.FA_ERROR_INVALID_VALUE
    assert bwd(N=0, Nk=0, q=None, ws=None, ws_bytes=0) == fa.FA_SUCCESS
    assert bwd(N=0, Nk=16, dk=None) == fa.FA_ERROR_INVALID_VALUE


def test_forward_grid_too_large_is_rejected():
    assert fwd(B=65535, H=65535, N=1 << 20) == fa.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [
    dict(dtype=9), dict(B=-1), dict(scale=0.0), dict(scale=math.nan), dict(causal=3),
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(do=None), dict(lse=None),
    dict(dq=None), dict(dk=None), dict(dv=None), dict(ws=None),
    dict(dq=MIS), dict(do=MIS), dict(ws=MIS), dict(lens=A + 1),
    dict(ws_bytes=16 * 4 - 1),
])
def test_backward_rejects_invalid_arguments(kw):
    assert bwd(**kw) == fa.FA_ERROR_INVALID_VALUE


def test_backward_unsupported_and_workspace_size():
    assert bwd(dtype=F32, d=160) == fa.FA_ERROR_UNSUPPORTED
    assert bwd(dtype=F32, d=512) == fa.FA_ERROR_UNSUPPORTED
    assert bwd(d=224) == fa.FA_ERROR_UNSUPPORTED
    assert bwd(d=80) == fa.FA_ERROR_UNSUPPORTED
    assert bwd(dtype=F16, d=160) == fa.FA_ERROR_UNSUPPORTED
    assert bwd(dtype=F16, B=0, q=None, ws=None, ws_bytes=0) == fa.FA_SUCCESS
    assert bwd(dtype=3) == fa.FA_ERROR_INVALID_VALUE
    assert fa.fa_backward_workspace_size(BF16, 2, 32, 8192, 128) == 2 * 32 * 8192 * 4
    assert fa.fa_backward_workspace_size(BF16, 0, 32, 8192, 128) == 0
    assert fa.fa_backward_workspace_size(BF16, -1, 32, 8192, 128) == 0
    assert bwd(B=0, q=None, ws=None, ws_bytes=0) == fa.FA_SUCCESS


def fwd_varlen(dtype=BF16, B=2, H=1, tq=40, tk=40, mq=20, mk=20, d=128, q=A, k=A, v=A, cq=A,
               ck=A, scale=0.1, causal=0, o=A, lse=A):
    return fa.fa_forward_varlen(dtype, B, H, tq, tk, mq, mk, d, q, k, v, cq, ck, scale, causal, o,
                                lse, None)


def bwd_varlen(dtype=BF16, B=2, H=1, tq=40, tk=40, mq=20, mk=20, d=128, scale=0.1, causal=0,
               ws=A, ws_bytes=1 << 20, **ptrs):
    p = dict(q=A, k=A, v=A, o=A, do=A, lse=A, cq=A, ck=A, dq=A, dk=A, dv=A)
    p.update(ptrs)
    return fa.fa_backward_varlen(dtype, B, H, tq, tk, mq, mk, d, p["q"], p["k"], p["v"], p["o"],
                                 p["do"], p["lse"], p["cq"], p["ck"], scale, causal, p["dq"],
                                 p["dk"], p["dv"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(dtype=5), dict(B=-1), dict(H=-1), dict(tq=-1), dict(tk=-1), dict(mq=-1), dict(mk=-1),
    dict(d=0), dict(scale=0.0), dict(scale=math.inf), dict(causal=2),
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None), dict(cq=None),
    dict(ck=None), dict(q=MIS), dict(o=MIS), dict(lse=MIS), dict(cq=A + 2), dict(ck=A + 1),
])
def test_forward_varlen_rejects_invalid_arguments(kw):
    assert fwd_varlen(**kw) == fa.FA_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [
    dict(dtype=5), dict(B=-1), dict(tk=-1), dict(mq=-1), dict(scale=math.nan), dict(causal=-1),
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(do=None), dict(lse=None),
    dict(cq=None), dict(ck=None), dict(dq=None), dict(dk=None), dict(dv=None), dict(ws=None),
    dict(dk=MIS), dict(ws=MIS), dict(cq=A + 2), dict(ws_bytes=40 * 4 - 1),
])
def test_backward_varlen_rejects_invalid_arguments(kw):
    assert bwd_varlen(**kw) == fa.FA_ERROR_INVALID_VALUE


def test_varlen_empty_unsupported_and_limits():
    none = dict(q=None, k=None, v=None, o=None, lse=None, cq=None, ck=None)
    for B, H in ((0, 4), (3, 0)):
        assert fwd_varlen(B=B, H=H, **none) == fa.FA_SUCCESS
    # no query rows: nothing to write, but the offsets are still required
    assert fwd_varlen(tq=0, q=None, o=None, lse=None) == fa.FA_SUCCESS
    assert fwd_varlen(mq=0, q=None, o=None, lse=None) == fa.FA_SUCCESS
    assert fwd_varlen(tq=0, cq=None) == fa.FA_ERROR_INVALID_VALUE
    # queries without keys still write empty rows, so o and lse are required
    assert fwd_varlen(tk=0, k=None, v=None, lse=None) == fa.FA_ERROR_INVALID_VALUE
    assert fwd_varlen(d=160) == fa.FA_ERROR_UNSUPPORTED
    assert fwd_varlen(dtype=F32, d=512) == fa.FA_ERROR_UNSUPPORTED
    assert bwd_varlen(d=224) == fa.FA_ERROR_UNSUPPORTED
    # one sequence's head must stay under 2^31 bytes
    assert fwd_varlen(mq=1 << 23, tq=1 << 23) == fa.FA_ERROR_UNSUPPORTED
    assert fwd(N=1 << 23) == fa.FA_ERROR_UNSUPPORTED
    assert fwd(dtype=F32, N=1 << 22) == fa.FA_ERROR_UNSUPPORTED
    assert bwd(N=16, Nk=1 << 23) == fa.FA_ERROR_UNSUPPORTED
    # backward: a side without rows needs no buffers
    assert bwd_varlen(tq=0, tk=0, q=None, k=None, ws=None, ws_bytes=0) == fa.FA_SUCCESS
    # keys without queries still write zero dK, dV rows: those are required
    assert bwd_varlen(tq=0, q=None, o=None, do=None, lse=None, dq=None, ws=None, ws_bytes=0,
                      dk=None) == fa.FA_ERROR_INVALID_VALUE
    assert bwd_varlen(tk=0, k=None, v=None, dk=None, dv=None, dq=None) == \
        fa.FA_ERROR_INVALID_VALUE
    assert fwd_varlen(B=1 << 20, H=1 << 10, mq=1 << 16) == fa.FA_ERROR_INVALID_VALUE


def fwd_fp8(B=1, H=1, N=16, Nk=16, d=128, q=A, k=A, v=A, lens=None, scale=0.1, qd=0.5, kd=0.5,
            vd=0.5, causal=0, o=A, lse=A):
    return fa.fa_forward_fp8(B, H, N, Nk, d, q, k, v, lens, scale, qd, kd, vd, causal, o, lse,
                             None)


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(N=-1), dict(Nk=-1), dict(d=0), dict(scale=0.0), dict(scale=math.nan),
    dict(qd=0.0), dict(kd=-1.0), dict(vd=math.inf), dict(qd=math.nan), dict(causal=2),
    dict(scale=1e30, qd=1e30, kd=1e30),
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(q=MIS), dict(k=MIS), dict(o=MIS), dict(lse=MIS), dict(lens=A + 2),
])
def test_forward_fp8_rejects_invalid_arguments(kw):
    assert fwd_fp8(**kw) == fa.FA_ERROR_INVALID_VALUE


def test_forward_fp8_unsupported_and_empty():
    for d in (64, 96, 256):
        assert fwd_fp8(d=d) == fa.FA_ERROR_UNSUPPORTED
    assert fwd_fp8(N=0, q=None, k=None, v=None, o=None, lse=None) == fa.FA_SUCCESS
    assert fwd_fp8(B=0, q=None, o=None, lse=None) == fa.FA_SUCCESS
    assert fwd_fp8(N=8, Nk=0, k=None, v=None, o=None) == fa.FA_ERROR_INVALID_VALUE
    assert fwd_fp8(B=65535, H=65535, N=1 << 20, Nk=1 << 20) == fa.FA_ERROR_INVALID_VALUE


def test_torch_wrappers_validate_before_calling():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 128, dtype=torch.float64)
    with pytest.raises(fa.FAError) as e:
        fa.forward(q, q, q)
    assert e.value.status == fa.FA_ERROR_UNSUPPORTED
    with pytest.raises(ValueError):
        fa.forward(q[0], q[0], q[0])
    b = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(b, b.float(), b)


def test_backward_wrappers_reject_strided_q():
    """A q view that is not dense (here sliced along N from a larger buffer)
    must be refused before any launch, even when every other tensor and dq
    are dense: the kernels index q as a contiguous [B][H][N][d] tensor."""
    torch = pytest.importorskip("torch")
    big = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    q = big[:, :, ::2]
    dense = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 4, dtype=torch.float32)
    assert not q.is_contiguous() and q.shape == dense.shape
    for fn in (fa.backward, fa.backward_phases):
        with pytest.raises(ValueError, match="q must be contiguous"):
            fn(q, dense, dense, dense, dense, lse, dq=dense.clone(), dk=dense.clone(),
               dv=dense.clone())
        with pytest.raises(ValueError):
            fn(dense[0], dense[0], dense[0], dense[0], dense[0], lse)
    with pytest.raises(ValueError, match="delta"):
        fa.backward_phases(dense, dense, dense, dense, dense, lse, delta=lse[0])


def test_backward_phase_entry_points_validate():
    pre = lambda o=A, do=A, delta=A, **kw: fa.fa_backward_preprocess(
        kw.get("dtype", BF16), kw.get("B", 1), kw.get("H", 1), kw.get("N", 16), kw.get("d", 128),
        o, do, delta, None)
    assert pre(o=None) == fa.FA_ERROR_INVALID_VALUE
    assert pre(delta=MIS) == fa.FA_ERROR_INVALID_VALUE
    assert pre(d=160) == fa.FA_ERROR_UNSUPPORTED
    assert pre(dtype=F32, d=224) == fa.FA_ERROR_UNSUPPORTED
    assert pre(N=0, o=None, do=None, delta=None) == fa.FA_SUCCESS

    def dkdv(q=A, dk=A, dv=A, delta=A, scale=0.1, causal=0, d=128, N=16, Nk=None):
        Nk = N if Nk is None else Nk
        return fa.fa_backward_dkdv(BF16, 1, 1, N, Nk, d, q, A, A, A, A, delta, None, scale,
                                   causal, dk, dv, None)

    def dq(q=A, out=A, delta=A, scale=0.1, causal=0, d=128, N=16, Nk=None):
        Nk = N if Nk is None else Nk
        return fa.fa_backward_dq(BF16, 1, 1, N, Nk, d, q, A, A, A, A, delta, None, scale,
                                 causal, out, None)

    for f in (dkdv, dq):
        assert f(q=None) == fa.FA_ERROR_INVALID_VALUE
        assert f(delta=None) == fa.FA_ERROR_INVALID_VALUE
        assert f(scale=-1.0) == fa.FA_ERROR_INVALID_VALUE
        assert f(causal=5) == fa.FA_ERROR_INVALID_VALUE
        assert f(d=80) == fa.FA_ERROR_UNSUPPORTED
        assert f(N=0, q=None, delta=None) == fa.FA_SUCCESS
        assert f(Nk=-1) == fa.FA_ERROR_INVALID_VALUE
    # keys without queries still have dK/dV rows; queries without keys, dQ rows
    assert dkdv(N=0, Nk=16, dk=None) == fa.FA_ERROR_INVALID_VALUE
    assert dq(N=16, Nk=0, out=None) == fa.FA_ERROR_INVALID_VALUE
    # a launch whose output has no rows does nothing, whatever the pointers
    assert dkdv(N=16, Nk=0, q=None, dk=None, dv=None) == fa.FA_SUCCESS
    assert dq(N=0, Nk=16, q=None, out=None) == fa.FA_SUCCESS
    assert dkdv(dk=None) == fa.FA_ERROR_INVALID_VALUE
    assert dkdv(dv=MIS) == fa.FA_ERROR_INVALID_VALUE
    assert dq(out=None) == fa.FA_ERROR_INVALID_VALUE


def dec(dtype=BF16, B=1, H=1, N=16, d=128, q=A, k=A, v=A, lens=None, scale=0.1, o=A, lse=A,
        ws=A, ws_bytes=1 << 20):
    return fa.fa_decode(dtype, B, H, N, d, q, k, v, lens, scale, o, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None), dict(ws=None),
    dict(q=MIS), dict(v=MIS), dict(o=MIS), dict(ws=MIS), dict(lens=A + 1),
    dict(scale=0.0), dict(scale=float("nan")), dict(B=-1), dict(d=0),
    dict(ws_bytes=16), dict(N=(1 << 24) + 1),
])
def test_decode_rejects_invalid_arguments(kw):
    assert dec(**kw) == fa.FA_ERROR_INVALID_VALUE


def test_decode_unsupported_and_empty():
    assert dec(d=160) == fa.FA_ERROR_UNSUPPORTED
    assert dec(dtype=F32, d=512) == fa.FA_ERROR_UNSUPPORTED
    assert dec(B=0, q=None, k=None, v=None, o=None, lse=None, ws=None, ws_bytes=0) == fa.FA_SUCCESS
    assert dec(N=0, q=None, ws=None, ws_bytes=0) == fa.FA_SUCCESS
    assert dec(dtype=F16, d=224) == fa.FA_ERROR_UNSUPPORTED
    assert dec(dtype=F16, B=0, q=None, k=None, v=None, o=None, lse=None, ws=None,
               ws_bytes=0) == fa.FA_SUCCESS


def test_decode_workspace_follows_the_split_plan():
    # B*H = 256 rows of 8192 keys: 32 parts of 256 keys, (d + 1) floats per part
    assert fa.fa_decode_workspace_size(BF16, 8, 32, 8192, 128) == 8 * 32 * 32 * 129 * 4
    # one short row: one part
    assert fa.fa_decode_workspace_size(BF16, 1, 1, 100, 128) == 129 * 4
    assert fa.fa_decode_workspace_size(BF16, 0, 1, 100, 128) == 0
    for B, H, N in [(1, 1, 1), (1, 32, 8192), (3, 5, 777), (64, 64, 65536), (1, 1, 1 << 24),
                    (2, 2, 4097), (1000, 8, 300)]:
        parts = fa.fa_decode_workspace_size(BF16, B, H, N, 64) // (B * H * 65 * 4)
        assert 1 <= parts <= 4096
        assert parts * 4096 >= N                       # no part holds more than 4096 keys
        assert parts <= max(1, -(-N // 64))            # parts hold at least 64 keys


def test_merge_states_validates():
    m = lambda dtype=F32, rows=4, parts=3, d=128, op=A, lp=A, o=A, lse=A: fa.fa_merge_states(
        dtype, rows, parts, d, op, lp, o, lse, None)
    assert m(op=None) == fa.FA_ERROR_INVALID_VALUE
    assert m(lp=None) == fa.FA_ERROR_INVALID_VALUE
    assert m(o=None) == fa.FA_ERROR_INVALID_VALUE
    assert m(o=MIS) == fa.FA_ERROR_INVALID_VALUE
    assert m(lse=MIS) == fa.FA_ERROR_INVALID_VALUE
    assert m(parts=0) == fa.FA_ERROR_INVALID_VALUE
    assert m(parts=4097) == fa.FA_ERROR_INVALID_VALUE
    assert m(rows=-1) == fa.FA_ERROR_INVALID_VALUE
    assert m(d=160) == fa.FA_ERROR_UNSUPPORTED
    assert m(rows=0, op=None, lp=None, o=None) == fa.FA_SUCCESS


def test_decode_torch_wrapper_validates_before_calling():
    torch = pytest.importorskip("torch")
    k = torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.decode(torch.zeros(1, 2, 64, dtype=torch.bfloat16), k, k)
    with pytest.raises(ValueError):
        fa.decode(torch.zeros(1, 2, 128, dtype=torch.float32), k, k)
    with pytest.raises(ValueError):
        fa.merge_states(torch.zeros(2, 3, 128), torch.zeros(2, 4))
