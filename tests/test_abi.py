"""C-ABI boundary checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before enqueuing anything."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_group_amd as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")
FAKE = ctypes.c_void_p(0x10000)     # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_(?:moe|dense)_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(bm.C_FUNCTIONS)
    L = bm.lib()
    for n in names:
        assert hasattr(L, n), n
    assert bm.abi_version() == 5


def test_status_strings():
    for s in range(5):
        assert bm.status_string(s).startswith("BEAM_")
    assert "unknown" in bm.status_string(99)


def beam(**kw):
    return bm.make_config(**kw)


def test_workspace_size_and_map():
    c = beam()
    n16 = bm.beam_moe_workspace_size(c, 16)
    n4k = bm.beam_moe_workspace_size(c, 4096)
    assert 0 < n16 < n4k
    m = bm.beam_moe_workspace_map(c, 4096)
    assert m["total"] == n4k
    offs = [m[k] for k in ("logits", "expert_count", "expert_off", "row_of_pair", "pair_of_row", "hidden",
                           "expert_out")]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    # expert outputs [T*K, H] BF16 are the largest region
    assert n4k - m["expert_out"] >= 4096 * 8 * 5120 * 2
    assert bm.beam_moe_workspace_size(c, -1) == 0
    assert bm.beam_moe_workspace_size(beam(n_groups=3), 16) == 0
    # E4M3 activation regions: present for 8-bit weights, empty for BF16
    assert m["x_q_scale"] == m["x_q"] and m["h_q_scale"] == m["h_q"]
    f = bm.beam_moe_workspace_map(beam(weight_dtype=bm.BEAM_DTYPE_FP8_E4M3), 4096)
    assert f["x_q_scale"] - f["x_q"] >= 4096 * 5120 and f["h_q_scale"] - f["h_q"] >= 4096 * 8 * 2560
    assert all(f[k] % 256 == 0 and f[k] < f["total"] for k in ("x_q", "x_q_scale", "h_q", "h_q_scale"))


@pytest.mark.parametrize("kw", [dict(n_groups=3), dict(n_groups=256), dict(topk_groups=9), dict(topk=0),
                                dict(topk=33), dict(topk_groups=1, topk=33), dict(n_experts=512),
                                dict(n_experts=1), dict(hidden=0), dict(routed_scale=float("nan")),
                                dict(act_dtype=7), dict(fp8_scale_kind=2), dict(fp8_scale_kind=-1)])
def test_invalid_config_rejected(kw):
    c = beam(**kw)
    st = bm.lib().beam_moe_forward(ctypes.byref(c), 16, FAKE, FAKE, None, None, FAKE, None, FAKE, None, FAKE,
                                   None, None, FAKE, 1 << 40, None)
    assert st == bm.BEAM_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(act_dtype=bm.BEAM_DTYPE_F32, weight_dtype=bm.BEAM_DTYPE_BF16),
                                dict(hidden=5000), dict(inter=100), dict(n_experts=96, n_groups=32),
                                dict(hidden=384),     # the prefill down GEMM tiles H by 256
                                dict(weight_dtype=bm.BEAM_DTYPE_FP8_E4M3, fp8_block=64)])
def test_unsupported_config(kw):
    c = beam(**kw)
    st = bm.lib().beam_moe_forward(ctypes.byref(c), 16, FAKE, FAKE, None, None, FAKE, None, FAKE, None, FAKE,
                                   None, None, FAKE, 1 << 40, None)
    assert st == bm.BEAM_ERR_UNSUPPORTED


def test_argument_errors_before_any_launch():
    c = beam()
    L = bm.lib()
    fwd = lambda T, x, y, ws, nb, w13=FAKE, s13=None: L.beam_moe_forward(
        ctypes.byref(c), T, x, FAKE, None, None, w13, s13, FAKE, None, y, None, None, ws, nb, None)
    assert fwd(0, None, None, None, 0) == bm.BEAM_OK                   # T = 0: no-op
    assert fwd(-1, FAKE, FAKE, FAKE, 1 << 40) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, None, FAKE, FAKE, 1 << 40) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, FAKE, None, FAKE, 1 << 40) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, FAKE, FAKE, FAKE, 1 << 40, w13=None) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, FAKE, FAKE, FAKE, 1 << 40, s13=FAKE) == bm.BEAM_ERR_INVALID_ARG   # scale with BF16
    assert fwd(16, ctypes.c_void_p(0x10008), FAKE, FAKE, 1 << 40) == bm.BEAM_ERR_INVALID_ARG  # misaligned
    need = bm.beam_moe_workspace_size(c, 16)
    assert fwd(16, FAKE, FAKE, FAKE, need - 1) == bm.BEAM_ERR_WORKSPACE
    assert fwd(16, FAKE, FAKE, None, need) == bm.BEAM_ERR_WORKSPACE
    # FP8 weights need both scale arrays
    c8 = beam(weight_dtype=bm.BEAM_DTYPE_FP8_E4M3)
    st = L.beam_moe_forward(ctypes.byref(c8), 16, FAKE, FAKE, None, None, FAKE, None, FAKE, FAKE, FAKE, None,
                            None, FAKE, 1 << 40, None)
    assert st == bm.BEAM_ERR_INVALID_ARG


def test_mxfp4_needs_scales_and_bounded_k_above_the_streaming_range():
    c = beam(weight_dtype=bm.BEAM_DTYPE_MXFP4)
    L = bm.lib()
    fwd = lambda T, s13, s2: L.beam_moe_forward(ctypes.byref(c), T, FAKE, FAKE, None, None, FAKE, s13, FAKE, s2,
                                                FAKE, None, None, FAKE, 1 << 40, None)
    assert fwd(16, None, FAKE) == bm.BEAM_ERR_INVALID_ARG          # both scale arrays required
    assert bm.beam_moe_workspace_size(c, 4096) > 0
    # above the streaming range a tile's weight scales must fit in LDS (K <= 8192)
    c = beam(weight_dtype=bm.BEAM_DTYPE_MXFP4, hidden=10240)
    assert fwd(257, FAKE, FAKE) == bm.BEAM_ERR_UNSUPPORTED


def test_route_and_sublayer_argument_errors():
    c = beam()
    L = bm.lib()
    assert L.beam_moe_route(ctypes.byref(c), 16, FAKE, FAKE, None, None, None, FAKE, FAKE, 1 << 40,
                            None) == bm.BEAM_ERR_INVALID_ARG
    assert L.beam_moe_route(ctypes.byref(c), 0, None, None, None, None, None, None, None, 0,
                            None) == bm.BEAM_OK
    sub = lambda cfg, k, ws_bytes: L.beam_moe_sublayer_forward(
        ctypes.byref(cfg), 16, FAKE, None, None, k, FAKE, None, None, FAKE, None, FAKE, None, None, None, None,
        FAKE, ws_bytes, None)
    assert sub(c, 1, 1 << 40) == bm.BEAM_ERR_INVALID_ARG                 # step k must be >= 2
    assert sub(beam(act_dtype=bm.BEAM_DTYPE_F32, weight_dtype=bm.BEAM_DTYPE_F32), 10,
               1 << 40) == bm.BEAM_ERR_UNSUPPORTED
    assert sub(c, 10, 16) == bm.BEAM_ERR_WORKSPACE


def test_fp8_reduction_bound_above_the_streaming_range():
    """FP8 tiles keep the K-block scale codes of one reduction in LDS: K <= 32768 where a
    GEMM runs tiled (the down GEMM, reducing over inter, from 104 tokens on)."""
    c = beam(weight_dtype=bm.BEAM_DTYPE_FP8_E4M3, inter=32768 + 128)
    fwd = lambda T: bm.lib().beam_moe_forward(ctypes.byref(c), T, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE,
                                              FAKE, None, None, FAKE, 1 << 40, None)
    assert fwd(104) == bm.BEAM_ERR_UNSUPPORTED
    assert fwd(257) == bm.BEAM_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# dense MLP entry points
# ---------------------------------------------------------------------------
def test_dense_workspace_and_config_checks():
    c = bm.make_dense_config()
    n16, n4k = bm.beam_dense_workspace_size(c, 16), bm.beam_dense_workspace_size(c, 4096)
    assert 0 < n16 < n4k
    # h [T, I] BF16 and the [T, H] down output at least; no router regions
    assert n4k >= 4096 * (20480 + 5120) * 2
    assert n4k < bm.beam_moe_workspace_size(bm.make_config(), 4096) * 2
    # split-K partial sums in the streaming range: up to 8 FP32 slices of [T, H]
    assert n16 >= 8 * 16 * 5120 * 4
    assert bm.beam_dense_workspace_size(c, -1) == 0
    assert bm.beam_dense_workspace_size(bm.make_dense_config(hidden=0), 16) == 0
    # the router fields are not read
    odd = bm.make_dense_config()
    odd.n_experts, odd.n_groups, odd.topk = 0, 0, 0
    assert bm.beam_dense_workspace_size(odd, 16) == n16


@pytest.mark.parametrize("kw,status", [(dict(hidden=0), bm.BEAM_ERR_INVALID_ARG),
                                       (dict(act_dtype=9), bm.BEAM_ERR_INVALID_ARG),
                                       (dict(norm_eps=float("inf")), bm.BEAM_ERR_INVALID_ARG),
                                       (dict(fp8_scale_kind=5), bm.BEAM_ERR_INVALID_ARG),
                                       (dict(hidden=384), bm.BEAM_ERR_UNSUPPORTED),
                                       (dict(inter=100), bm.BEAM_ERR_UNSUPPORTED),
                                       (dict(act_dtype=bm.BEAM_DTYPE_F32), bm.BEAM_ERR_UNSUPPORTED)])
def test_dense_config_errors(kw, status):
    c = bm.make_dense_config(**kw)
    st = bm.lib().beam_dense_forward(ctypes.byref(c), 16, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 1 << 40, None)
    assert st == status


def test_dense_argument_errors_before_any_launch():
    c = bm.make_dense_config()
    L = bm.lib()
    fwd = lambda T, x, y, ws, nb, w13=FAKE, s13=None, cfg=c: L.beam_dense_forward(
        ctypes.byref(cfg), T, x, w13, s13, FAKE, None, y, ws, nb, None)
    assert fwd(0, None, None, None, 0) == bm.BEAM_OK
    assert fwd(-1, FAKE, FAKE, FAKE, 1 << 40) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, None, FAKE, FAKE, 1 << 40) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, FAKE, None, FAKE, 1 << 40) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, FAKE, FAKE, FAKE, 1 << 40, w13=None) == bm.BEAM_ERR_INVALID_ARG
    assert fwd(16, FAKE, FAKE, FAKE, 1 << 40, s13=FAKE) == bm.BEAM_ERR_INVALID_ARG
    need = bm.beam_dense_workspace_size(c, 16)
    assert fwd(16, FAKE, FAKE, FAKE, need - 1) == bm.BEAM_ERR_WORKSPACE
    # MXFP4 above the dense streaming range (16 tokens): the tiled kernels stage a K
    # slice's weight scales in LDS (at most 8192 long), so the down GEMM of width 20480
    # runs in 4 slices; hidden must stay <= 8192 and the width split into whole slices
    c4 = bm.make_dense_config(weight_dtype=bm.BEAM_DTYPE_MXFP4)
    mx = lambda cfg, T, nb: L.beam_dense_forward(ctypes.byref(cfg), T, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                 nb, None)
    assert mx(c4, 33, 16) == bm.BEAM_ERR_WORKSPACE
    assert mx(bm.make_dense_config(weight_dtype=bm.BEAM_DTYPE_MXFP4, hidden=10240), 33, 1 << 40) == \
        bm.BEAM_ERR_UNSUPPORTED
    assert mx(bm.make_dense_config(weight_dtype=bm.BEAM_DTYPE_MXFP4, inter=20608), 33, 1 << 40) == \
        bm.BEAM_ERR_UNSUPPORTED
    assert mx(bm.make_dense_config(weight_dtype=bm.BEAM_DTYPE_MXFP4, inter=20608), 16, 16) == \
        bm.BEAM_ERR_WORKSPACE
    sub = lambda cfg, k, nb: L.beam_dense_sublayer_forward(ctypes.byref(cfg), 16, FAKE, None, None, k, FAKE,
                                                           None, FAKE, None, None, FAKE, nb, None)
    assert sub(c, 1, 1 << 40) == bm.BEAM_ERR_INVALID_ARG
    assert sub(bm.make_dense_config(act_dtype=bm.BEAM_DTYPE_F32, weight_dtype=bm.BEAM_DTYPE_F32), 10,
               1 << 40) == bm.BEAM_ERR_UNSUPPORTED
    assert sub(c, 10, 16) == bm.BEAM_ERR_WORKSPACE


def test_noalloc_forward_refuses_beyond_the_static_scratch():
    """The no-allocation forward checks the workspace its call needs against the static
    scratch size on the host, before it looks up the scratch or enqueues anything."""
    L = bm.lib()
    c = beam()
    assert bm.beam_moe_workspace_size(c, 4096) > bm.NOALLOC_SCRATCH_BYTES
    call = lambda cfg, T: L.beam_moe_forward_noalloc(ctypes.byref(cfg), T, FAKE, FAKE, None, None, FAKE, None,
                                                     FAKE, None, FAKE, None, None, None)
    assert call(c, 4096) == bm.BEAM_ERR_WORKSPACE
    assert call(c, 0) == bm.BEAM_OK
    assert call(beam(n_groups=3), 16) == bm.BEAM_ERR_INVALID_ARG
    assert call(beam(hidden=5000), 16) == bm.BEAM_ERR_UNSUPPORTED
    # Beam's BF16 decode batch fits
    assert bm.beam_moe_workspace_size(c, 16) <= bm.NOALLOC_SCRATCH_BYTES
