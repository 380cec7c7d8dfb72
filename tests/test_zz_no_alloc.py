"""beam_moe_forward_noalloc -- the forward on the library's static per-device scratch
array, with no workspace argument -- against beam_moe_forward with a caller-owned
workspace, through the C ABI: calls in a row on the same device, each later one smaller
than the one before (the scratch keeps the previous call's contents), with BF16 and FP8
(amax / 448 block scales) experts.  The two entry points run the same kernels on the same
inputs, so outputs, ids and weights must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_mixture_experts_group_amd as bm
from beam_inputs import DT_BF16, DT_FP8, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("wdt", [DT_BF16, DT_FP8])
def test_noalloc_forward_matches_workspace_forward(wdt):
    w = Workload("noalloc", T=300, H=1024, I=512, E=64, G=8, Kg=4, K=8, weight_dtype=wdt, seed=5,
                 x_recipe="rms_normal")
    inp = make_inputs(w)
    cfg = bm.make_config(hidden=w.H, inter=w.I, n_experts=w.E, n_groups=w.G, topk_groups=w.Kg, topk=w.K,
                         weight_dtype=wdt)
    wr, w13, w2 = _dev(inp.w_router), _dev(inp.w13), _dev(inp.w2)
    s13 = _dev(inp.w13_scale) if inp.w13_scale is not None else None
    s2 = _dev(inp.w2_scale) if inp.w2_scale is not None else None
    x_all = _dev(inp.x)
    L = bm.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # tiled gate/up and down GEMMs; tiled gate/up with the streaming down GEMM; both streaming
    for T in (300, 40, 9):
        assert bm.beam_moe_workspace_size(cfg, T) <= bm.NOALLOC_SCRATCH_BYTES
        print(f"[case] noalloc dtype={wdt} T={T}", flush=True)
        x = x_all[:T].contiguous()
        ids_r = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
        wts_r = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
        y_r = bm.beam_moe_forward(cfg, x, wr, w13, w2, w13_scale=s13, w2_scale=s2, ids=ids_r, weights=wts_r)
        ids_n = torch.full((T, w.K), -1, dtype=torch.int32, device="cuda")
        wts_n = torch.full((T, w.K), -1.0, dtype=torch.float32, device="cuda")
        y_n = torch.zeros_like(x)
        st = L.beam_moe_forward_noalloc(ctypes.byref(cfg), T, _ptr(x), _ptr(wr), None, None, _ptr(w13), _ptr(s13),
                                        _ptr(w2), _ptr(s2), _ptr(y_n), _ptr(ids_n), _ptr(wts_n), stream)
        assert st == bm.BEAM_OK, bm.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(ids_n, ids_r)
        assert torch.equal(wts_n.view(torch.int32), wts_r.view(torch.int32))
        assert torch.equal(y_n.view(torch.int16), y_r.view(torch.int16))
    # too large for the static scratch: refused before anything is enqueued
    big = bm.make_config(weight_dtype=wdt)
    assert bm.beam_moe_workspace_size(big, 32768) > bm.NOALLOC_SCRATCH_BYTES
    assert L.beam_moe_forward_noalloc(ctypes.byref(big), 32768, _ptr(x_all), _ptr(wr), None, None, _ptr(w13),
                                      _ptr(s13), _ptr(w2), _ptr(s2), _ptr(y_n), None, None,
                                      stream) == bm.BEAM_ERR_WORKSPACE
