"""fa_backward_noalloc on the GPU: its workspace is the library's static
per-GPU array, so it must give exactly what fa_backward gives with a caller
workspace, call after call (the array keeps the previous call's contents),
for a smaller problem after a larger one, and refuse a problem that does not
fit before launching anything."""

import numpy as np
import pytest

import fa_inputs as fi
from tests.gpu_helpers import custom, device_inputs, lib, log_case, torch_cuda

pytestmark = pytest.mark.gpu


def _fwd_bwd_both(torch, fa, cfg, inputs):
    dev = device_inputs(torch, cfg, inputs)
    lens = dev["lengths"]
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=cfg.causal,
                        seqlens_k=lens)
    ref = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=cfg.scale,
                      causal=cfg.causal, seqlens_k=lens)
    outs = [torch.full_like(t, float("nan")) for t in ref]
    got = fa.backward_noalloc(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *outs,
                              scale=cfg.scale, causal=cfg.causal, seqlens_k=lens)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_backward_matches_backward_on_consecutive_calls(dtype):
    torch = torch_cuda()
    fa = lib()
    shapes = [dict(B=2, H=4, N=1000, d=128, causal=True),     # larger first
              dict(B=1, H=2, N=300, d=64, causal=False)]      # then smaller
    for i, shp in enumerate(shapes):
        cfg = custom(5, dtype=dtype, **shp)
        log_case(test="noalloc", call=i, dtype=dtype, **shp)
        inputs = fi.make_inputs(cfg, seed=40 + i)
        if i == 0:
            inputs["lengths"] = np.array([700, 1000], np.int32)
        ref, got = _fwd_bwd_both(torch, fa, cfg, inputs)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert not torch.isnan(b).any().item(), name
            assert torch.equal(a, b), f"{name} differs on call {i}"


def test_noalloc_backward_refuses_a_problem_beyond_its_workspace():
    torch = torch_cuda()
    fa = lib()
    rows = fa.FA_NOALLOC_SCRATCH_BYTES // 4
    q = torch.zeros(1, 1, 16, 128, dtype=torch.bfloat16, device="cuda")
    st = fa.fa_backward_noalloc(fa.FA_DTYPE_BF16, 1, 1, rows + 1, rows + 1, 128, q.data_ptr(),
                                q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                q.data_ptr(), None, 0.1, 0, q.data_ptr(), q.data_ptr(),
                                q.data_ptr(), None)
    assert st == fa.FA_ERROR_SCRATCH_LIMIT
