"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.  Routing ids and the permutation are compared bit for bit, FP32 weights within
1e-6 relative, layer outputs within the stated relative max-norm tolerance
(||y - y_ref||_inf / ||y_ref||_inf): 1e-5 FP32 layer, 2e-2 BF16 experts, 6e-2 FP8 experts.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_group_amd as bm
from beam_inputs import DT_BF16, DT_F32, DT_FP8, DT_MXFP4, DTYPE_NAMES, WORKLOADS
from conftest import gpu_inputs

pytestmark = pytest.mark.gpu

# MXFP4 weights are exact as stored on both sides; the GPU error is the E4M3 activation
# quantisation, as on the FP8 path
TOL = {DT_F32: 1e-5, DT_BF16: 2e-2, DT_FP8: 6e-2, DT_MXFP4: 6e-2}


def cfg_of(w):
    return bm.make_config(hidden=w.H, inter=w.I, n_experts=w.E, n_groups=w.G, topk_groups=w.Kg, topk=w.K,
                          routed_scale=w.alpha, act_dtype=w.act_dtype, weight_dtype=w.weight_dtype,
                          fp8_block=w.fp8_block, norm_eps=w.norm_eps)


def to_dev_x(w, x):
    if w.act_dtype == DT_F32:
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def x_f32(w, x):
    return x if w.act_dtype == DT_F32 else oracle.bf16_to_f32(x)


def bank_of(w, full):
    return oracle.ExpertBank(full.w13, full.w2, DTYPE_NAMES[w.weight_dtype], full.w13_scale, full.w2_scale,
                             w.fp8_block)


def dev_bias(bias):
    return None if bias is None else torch.from_numpy(bias).cuda()


def rel_inf(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def sample_tokens(T, n=16, seed=1):
    rs = np.random.default_rng(seed)
    base = {0, T - 1, T // 2}
    extra = rs.choice(T, size=min(T, n), replace=False)
    return np.array(sorted(base | set(int(t) for t in extra)))[:max(n, 3)]


def run_forward(w, dev, x, bias, select_bias=None):
    cfg = cfg_of(w)
    xd = to_dev_x(w, x)
    ids = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")
    ws = bm.alloc_workspace(cfg, w.T)
    y = bm.beam_moe_forward(cfg, xd, dev["w_router"], dev["w13"], dev["w2"], logit_bias=dev_bias(bias),
                            w13_scale=dev.get("w13_scale"), w2_scale=dev.get("w2_scale"), ids=ids, weights=wts,
                            ws=ws, select_bias=dev_bias(select_bias))
    torch.cuda.synchronize()
    return cfg, y, ids.cpu().numpy(), wts.cpu().numpy(), ws


def ws_region(ws, off, count, dtype):
    nbytes = count * np.dtype(dtype).itemsize
    return ws[off:off + nbytes].cpu().numpy().view(dtype)


def check_routing(w, ids, wts, ref_ids, ref_w):
    mism = int((ids != ref_ids).any(axis=1).sum())
    assert mism == 0, f"{mism} tokens with different expert ids"
    rel = np.abs(wts.astype(np.float64) - ref_w) / np.abs(ref_w)
    assert rel.max() <= 1e-6, rel.max()


def check_permutation(w, ws, ids):
    m = bm.beam_moe_workspace_map(cfg_of(w), w.T)
    P = w.T * w.K
    cnt = ws_region(ws, m["expert_count"], w.E, np.int32)
    off = ws_region(ws, m["expert_off"], w.E + 1, np.int32)
    rop = ws_region(ws, m["row_of_pair"], P, np.int32)
    por = ws_region(ws, m["pair_of_row"], P, np.int32)
    flat = ids.reshape(-1)
    assert np.array_equal(cnt, np.bincount(flat, minlength=w.E))
    assert off[0] == 0 and np.array_equal(np.diff(off), cnt)
    # stable order: rows of each expert consecutive, pairs ascending inside an expert
    assert np.array_equal(por, np.argsort(flat, kind="stable"))
    assert np.array_equal(rop[por], np.arange(P))


# ---------------------------------------------------------------------------
# tiny FP32 layer: everything checked, every token
# ---------------------------------------------------------------------------
def test_tiny_layer_full_parity():
    w, full, dev, x, bias = gpu_inputs("tiny_f32")
    print(f"[case] tiny_f32 T={w.T}", flush=True)
    cfg, y, ids, wts, ws = run_forward(w, dev, x, bias)
    ref = oracle.moe_forward(x_f32(w, x), full.w_router, bias, bank_of(w, full), w.G, w.Kg, w.K, w.alpha)
    check_routing(w, ids, wts, ref["ids"], ref["w"])
    m = bm.beam_moe_workspace_map(cfg, w.T)
    z = ws_region(ws, m["logits"], w.T * w.E, np.float32).reshape(w.T, w.E)
    assert np.array_equal(z, ref["logits"])            # logits bit for bit
    check_permutation(w, ws, ids)
    assert rel_inf(y.cpu().numpy().astype(np.float64), ref["y"]) <= TOL[DT_F32]


@pytest.mark.parametrize("T", [1, 5, 33, 100, 300])
def test_tiny_layer_ragged_T(T):
    w, full, dev, x, bias = gpu_inputs("tiny_f32", T)
    print(f"[case] tiny_f32 T={T}", flush=True)
    cfg, y, ids, wts, ws = run_forward(w, dev, x, bias)
    ref = oracle.moe_forward(x_f32(w, x), full.w_router, bias, bank_of(w, full), w.G, w.Kg, w.K, w.alpha)
    check_routing(w, ids, wts, ref["ids"], ref["w"])
    check_permutation(w, ws, ids)
    assert rel_inf(y.cpu().numpy().astype(np.float64), ref["y"]) <= TOL[DT_F32]


# ---------------------------------------------------------------------------
# selection-only expert bias (ranking on s + b, weights from s)
# ---------------------------------------------------------------------------
def test_select_bias_tiny_layer_full_parity():
    w, full, dev, x, bias = gpu_inputs("tiny_f32")
    sb = (np.random.default_rng(21).standard_normal(w.E) * 0.2).astype(np.float32)
    print(f"[case] tiny_f32 select bias T={w.T}", flush=True)
    cfg, y, ids, wts, ws = run_forward(w, dev, x, bias, select_bias=sb)
    ref = oracle.moe_forward(x_f32(w, x), full.w_router, bias, bank_of(w, full), w.G, w.Kg, w.K, w.alpha,
                             select_bias=sb)
    check_routing(w, ids, wts, ref["ids"], ref["w"])
    check_permutation(w, ws, ids)
    assert rel_inf(y.cpu().numpy().astype(np.float64), ref["y"]) <= TOL[DT_F32]
    ref0 = oracle.moe_forward(x_f32(w, x), full.w_router, bias, bank_of(w, full), w.G, w.Kg, w.K, w.alpha)
    assert not np.array_equal(ref0["ids"], ref["ids"])      # the bias does change the routing


@pytest.mark.parametrize("T", [16, 300, 4096])
def test_select_bias_beam_routing(T):
    """Beam-shaped routing with a random selection bias (chunk-parallel and tiled logits
    kernels) and with a dominant bias forcing two experts in each of four groups."""
    w, full, dev, x, bias = gpu_inputs("beam_prefill_t4096", T)
    cfg = cfg_of(w)
    xd = to_dev_x(w, x)
    x32 = x_f32(w, x)
    z = oracle.router_logits(x32, full.w_router, bias)
    S = w.E // w.G
    forced = np.array([g * S + j for g in (0, 2, 5, 7) for j in (3, 30)])
    dominant = np.zeros(w.E, np.float32)
    dominant[forced] = 8.0
    for name, sb in (("random", (np.random.default_rng(22).standard_normal(w.E) * 0.02).astype(np.float32)),
                     ("dominant", dominant)):
        print(f"[case] beam routing T={T} select bias {name}", flush=True)
        ids, wts = bm.beam_moe_route(cfg, xd, dev["w_router"], logit_bias=dev_bias(bias), select_bias=dev_bias(sb))
        torch.cuda.synchronize()
        rid, rw = oracle.route(z, w.G, w.Kg, w.K, w.alpha, select_bias=sb)
        check_routing(w, ids.cpu().numpy(), wts.cpu().numpy(), rid, rw)
        if name == "dominant":
            assert np.array_equal(np.sort(rid, axis=1), np.tile(np.sort(forced), (T, 1)))


def test_router_all_ties_and_duplicated_columns():
    """W_r = 0: every score ties (ids 0..K-1, weights alpha/K).  Duplicated W_r columns
    across groups: exact equal scores across groups resolved toward lower indices."""
    w, full, dev, x, bias = gpu_inputs("beam_decode_t16")
    print("[case] router ties", flush=True)
    cfg = cfg_of(w)
    xd = to_dev_x(w, x)
    zero = torch.zeros_like(dev["w_router"])
    ids, wts = bm.beam_moe_route(cfg, xd, zero)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == np.arange(w.K)).all()
    assert (wts.cpu().numpy() == np.float32(w.alpha / w.K)).all()
    wr = full.w_router.copy()
    S = w.E // w.G
    for g in range(1, w.G):
        wr[:, g * S:(g + 1) * S] = wr[:, 0:S]          # every group a copy of group 0
    ids, wts = bm.beam_moe_route(cfg, xd, torch.from_numpy(wr).cuda())
    torch.cuda.synchronize()
    z = oracle.router_logits(x_f32(w, x), wr)
    rid, rw = oracle.route(z, w.G, w.Kg, w.K, w.alpha)
    check_routing(w, ids.cpu().numpy(), wts.cpu().numpy(), rid, rw)
    assert (ids.cpu().numpy() < w.Kg * S).all()        # equal groups -> the lowest Kg groups


# ---------------------------------------------------------------------------
# Beam-shaped BF16 layer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,T", [("beam_decode_t16", None), ("beam_decode_t16", 1),
                                    ("beam_decode_t16", 17), ("beam_decode_t16", 32),
                                    ("beam_prefill_t4096", 33), ("beam_prefill_t4096", 55),
                                    ("beam_prefill_t4096", 56), ("beam_prefill_t4096", 256),
                                    ("beam_prefill_t4096", 257), ("beam_prefill_t4096", 1000),
                                    ("beam_prefill_t4096", None),
                                    ("beam_prefill_t4096", 4097), ("beam_skewed_t32768", None)])
def test_beam_bf16_layer(name, T):
    w, full, dev, x, bias = gpu_inputs(name, T)
    print(f"[case] {name} T={w.T}", flush=True)
    cfg, y, ids, wts, ws = run_forward(w, dev, x, bias)
    # routing of every token, bit for bit
    x32 = x_f32(w, x)
    z = oracle.router_logits(x32, full.w_router, bias)
    rid, rw = oracle.route(z, w.G, w.Kg, w.K, w.alpha)
    check_routing(w, ids, wts, rid, rw)
    m = bm.beam_moe_workspace_map(cfg, w.T)
    zg = ws_region(ws, m["logits"], w.T * w.E, np.float32).reshape(w.T, w.E)
    assert np.array_equal(zg, z)
    check_permutation(w, ws, ids)
    # layer output of every token up to T = 300 (every tile of the grid), else sampled
    tok = np.arange(w.T) if w.T <= 300 else sample_tokens(w.T)
    yref = oracle.moe_combine(x32[tok].astype(np.float64), rid[tok], rw[tok], bank_of(w, full))
    yg = y.float().cpu().numpy()[tok].astype(np.float64)
    err = rel_inf(yg, yref)
    print(f"[case] {name} T={w.T} rel_inf={err:.3e}", flush=True)
    assert err <= TOL[w.weight_dtype]


def test_beam_bf16_intermediates_and_determinism():
    """SwiGLU activations (hidden) of sampled rows against the oracle's, and two runs
    giving bit-identical outputs."""
    w, full, dev, x, bias = gpu_inputs("beam_prefill_t4096")
    print("[case] intermediates T=4096", flush=True)
    cfg, y1, ids, wts, ws = run_forward(w, dev, x, bias)
    _, y2, _, _, _ = run_forward(w, dev, x, bias)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    m = bm.beam_moe_workspace_map(cfg, w.T)
    P = w.T * w.K
    por = ws_region(ws, m["pair_of_row"], P, np.int32)
    hid = ws_region(ws, m["hidden"], P * w.I, np.uint16).reshape(P, w.I)
    rows = np.random.default_rng(3).choice(P, 24, replace=False)
    x32 = x_f32(w, x).astype(np.float64)
    bank = bank_of(w, full)
    errs = []
    for r in rows:
        p = int(por[r]); t, i = divmod(p, w.K)
        w13, _ = bank.expert(int(ids[t, i]))
        g = w13[:w.I] @ x32[t]; u = w13[w.I:] @ x32[t]
        a = oracle.silu(g) * u
        errs.append(rel_inf(oracle.bf16_to_f32(hid[r]).astype(np.float64), a))
    assert max(errs) <= 2e-2, max(errs)


# ---------------------------------------------------------------------------
# FP8 sublayer
# ---------------------------------------------------------------------------
def test_fp8_sublayer():
    w, full, dev, x, bias = gpu_inputs("beam_sublayer_fp8_t8192")
    print(f"[case] sublayer fp8 T={w.T}", flush=True)
    cfg = cfg_of(w)
    h = to_dev_x(w, x)
    moe_out = torch.empty_like(h)
    ids = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")
    bm.beam_moe_sublayer_forward(cfg, h, w.step_k, dev["w_router"], dev["w13"], dev["w2"],
                                 w13_scale=dev["w13_scale"], w2_scale=dev["w2_scale"], moe_out=moe_out, ids=ids,
                                 weights=wts)
    torch.cuda.synchronize()
    h32 = oracle.bf16_to_f32(x)
    tok = sample_tokens(w.T)
    ref = oracle.sublayer_forward(h32, None, None, w.step_k, w.norm_eps, full.w_router, bias, bank_of(w, full),
                                  w.G, w.Kg, w.K, w.alpha, token_subset=tok)
    check_routing(w, ids.cpu().numpy(), wts.cpu().numpy(), ref["ids"], ref["w"])
    e_moe = rel_inf(moe_out.float().cpu().numpy()[tok].astype(np.float64), ref["y"])
    e_h = rel_inf(h.float().cpu().numpy()[tok].astype(np.float64), ref["h_new"])
    print(f"[case] sublayer fp8 moe rel_inf={e_moe:.3e} h rel_inf={e_h:.3e}", flush=True)
    assert e_moe <= TOL[DT_FP8]
    assert e_h <= TOL[DT_FP8]


@pytest.mark.parametrize("T", [16, 17, 100, 104, 200, 700])
def test_fp8_forward(T):
    """FP8 experts through beam_moe_forward at the crossovers: both GEMMs streaming (T =
    16), LDS-tiled gate/up with the streaming down GEMM (17, 100), both tiled with mostly
    partial tiles (104, 200, 700)."""
    w0, full, dev, _, bias = gpu_inputs("beam_sublayer_fp8_t8192")
    from dataclasses import replace
    from beam_inputs import token_inputs, to_bf16_bits
    w = replace(w0, T=T, sublayer=False, x_recipe="rms_normal")
    x = to_bf16_bits(token_inputs(w))
    print(f"[case] fp8 forward T={T}", flush=True)
    cfg, y, ids, wts, ws = run_forward(w, dev, x, None)
    x32 = oracle.bf16_to_f32(x)
    z = oracle.router_logits(x32, full.w_router, None)
    rid, rw = oracle.route(z, w.G, w.Kg, w.K, w.alpha)
    check_routing(w, ids, wts, rid, rw)
    check_permutation(w, ws, ids)
    tok = np.arange(T) if T <= 300 else sample_tokens(T)
    yref = oracle.moe_combine(x32[tok].astype(np.float64), rid[tok], rw[tok], bank_of(w, full))
    err = rel_inf(y.float().cpu().numpy()[tok].astype(np.float64), yref)
    print(f"[case] fp8 forward T={T} rel_inf={err:.3e}", flush=True)
    assert err <= TOL[DT_FP8]


# ---------------------------------------------------------------------------
# MXFP4 experts (E2M1 weights with E8M0 block scales, E4M3 activations)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,T", [("beam_decode_mxfp4_t16", None), ("beam_decode_mxfp4_t16", 200),
                                    ("beam_decode_mxfp4_t16", 700), ("beam_prefill_mxfp4_t4096", None)])
def test_mxfp4_forward(name, T):
    """MXFP4 experts through beam_moe_forward: streaming kernels up to 256 tokens (16 or
    32 rows per pass), LDS-tiled kernels above, against the oracle on the stored FP4
    weights (every token up to 300, else sampled tokens)."""
    w, full, dev, x, bias = gpu_inputs(name, T)
    T = w.T
    print(f"[case] mxfp4 forward T={T}", flush=True)
    cfg, y, ids, wts, ws = run_forward(w, dev, x, bias)
    x32 = oracle.bf16_to_f32(x)
    z = oracle.router_logits(x32, full.w_router, bias)
    rid, rw = oracle.route(z, w.G, w.Kg, w.K, w.alpha)
    check_routing(w, ids, wts, rid, rw)
    check_permutation(w, ws, ids)
    tok = np.arange(T) if T <= 300 else sample_tokens(T)
    yref = oracle.moe_combine(x32[tok].astype(np.float64), rid[tok], rw[tok], bank_of(w, full))
    err = rel_inf(y.float().cpu().numpy()[tok].astype(np.float64), yref)
    print(f"[case] mxfp4 forward T={T} rel_inf={err:.3e}", flush=True)
    assert err <= TOL[DT_MXFP4]



# ---------------------------------------------------------------------------
# dense SwiGLU MLP (the first decoder layers): one weight set, every token
# ---------------------------------------------------------------------------
_DENSE_BANK = {}


def dense_bank(w, full):
    """Float64 weights of the dense MLP, decoded once per weight dtype."""
    key = w.weight_dtype
    if key not in _DENSE_BANK:
        w13, w2 = bank_of(w, full).expert(0)
        _DENSE_BANK[key] = oracle.ExpertBank(w13[None], w2[None], "f32")
    return _DENSE_BANK[key]


def dense_cfg(w):
    return bm.make_dense_config(hidden=w.H, inter=w.I, act_dtype=w.act_dtype, weight_dtype=w.weight_dtype,
                                fp8_block=w.fp8_block, norm_eps=w.norm_eps)


@pytest.mark.parametrize("dt,T", [(DT_BF16, 16), (DT_BF16, 1), (DT_BF16, 17), (DT_BF16, 32), (DT_BF16, 33), (DT_BF16, 200),
                                  (DT_BF16, 700), (DT_BF16, 4096), (DT_FP8, 16), (DT_FP8, 200), (DT_FP8, 700),
                                  (DT_MXFP4, 16), (DT_MXFP4, 32), (DT_MXFP4, 200), (DT_MXFP4, 4096)])
def test_dense_forward(dt, T):
    """Dense MLP through beam_dense_forward: streaming kernels with both GEMMs split
    over K (T <= 16) and the LDS-tiled kernels, split over K while their tiles are few
    (T = 32, 33, 200, 700 ragged, 4096), against the oracle (every token up to 300, else
    sampled tokens)."""
    w, full, dev, x, _ = gpu_inputs("beam_dense_decode_t16", T, weight_dtype=dt)
    print(f"[case] dense forward {DTYPE_NAMES[dt]} T={T}", flush=True)
    cfg = dense_cfg(w)
    y = bm.beam_dense_forward(cfg, to_dev_x(w, x), dev["w13"], dev["w2"], w13_scale=dev.get("w13_scale"),
                              w2_scale=dev.get("w2_scale"))
    torch.cuda.synchronize()
    tok = np.arange(T) if T <= 300 else sample_tokens(T)
    ref = oracle.dense_forward(x_f32(w, x), dense_bank(w, full), token_subset=tok)
    got = y.float().cpu().numpy()[tok].astype(np.float64)
    err = rel_inf(got, ref["y"])
    print(f"[case] dense forward {DTYPE_NAMES[dt]} T={T} rel_inf={err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL[dt]


@pytest.mark.parametrize("dt,T", [(DT_BF16, 300), (DT_FP8, 16)])
def test_dense_sublayer(dt, T):
    """pre-norm -> dense MLP -> post-norm -> residual, h updated in place."""
    w, full, dev, x, _ = gpu_inputs("beam_dense_decode_t16", T, weight_dtype=dt, x_recipe="normal")
    print(f"[case] dense sublayer {DTYPE_NAMES[dt]} T={T}", flush=True)
    cfg = dense_cfg(w)
    rs = np.random.default_rng(11)
    g1 = (1 + 0.1 * rs.standard_normal(w.H)).astype(np.float32)
    g2 = (1 + 0.1 * rs.standard_normal(w.H)).astype(np.float32)
    h = to_dev_x(w, x)
    out = torch.empty_like(h)
    bm.beam_dense_sublayer_forward(cfg, h, w.step_k, dev["w13"], dev["w2"], pre_gain=torch.from_numpy(g1).cuda(),
                                   post_gain=torch.from_numpy(g2).cuda(), w13_scale=dev.get("w13_scale"),
                                   w2_scale=dev.get("w2_scale"), mlp_out=out)
    torch.cuda.synchronize()
    ref = oracle.dense_sublayer_forward(oracle.bf16_to_f32(x), g1, g2, w.step_k, w.norm_eps, dense_bank(w, full))
    e_y = rel_inf(out.float().cpu().numpy().astype(np.float64), ref["y"])
    e_h = rel_inf(h.float().cpu().numpy().astype(np.float64), ref["h_new"])
    print(f"[case] dense sublayer {DTYPE_NAMES[dt]} T={T} mlp rel_inf={e_y:.3e} h rel_inf={e_h:.3e}", flush=True)
    assert e_y <= TOL[dt] and e_h <= TOL[dt]


# ---------------------------------------------------------------------------
# limits of the configuration and degenerate routing
# ---------------------------------------------------------------------------
_EDGE = {
    # largest hidden size and top-k the kernels accept (H = 16384, K = 32)
    "max_hidden_topk": dict(H=16384, I=128, E=64, G=8, Kg=4, K=32),
    # one group: plain top-K over all experts
    "single_group": dict(H=512, I=256, E=64, G=1, Kg=1, K=6),
    # every group kept
    "all_groups_kept": dict(H=256, I=128, E=32, G=4, Kg=4, K=8),
    # K = 1: the weight is alpha exactly
    "k1": dict(H=128, I=64, E=16, G=4, Kg=2, K=1, act_dtype=DT_F32, weight_dtype=DT_F32),
    # the fewest experts: both picked
    "two_experts": dict(H=128, I=64, E=2, G=1, Kg=1, K=2, act_dtype=DT_F32, weight_dtype=DT_F32),
    # register-tiled router logits with 16-deep tiles (chunks of 16 hidden entries)
    "short_chunks": dict(H=1024, I=256, E=128, G=8, Kg=4, K=8),
    # FP8 reductions over more than 64 scale blocks (the 64-byte-stage GEMM with its
    # block scales in LDS): gate/up over H = 8448, down over I = 8448
    "fp8_long_hidden": dict(H=8448, I=256, E=16, G=4, Kg=2, K=4, weight_dtype=DT_FP8),
    "fp8_long_inter": dict(H=256, I=8448, E=16, G=4, Kg=2, K=4, weight_dtype=DT_FP8),
    # MXFP4 K slices longer than 6144 (the 64-byte-stage GEMM)
    "mxfp4_long_hidden": dict(H=6656, I=512, E=16, G=4, Kg=2, K=4, weight_dtype=DT_MXFP4),
    "mxfp4_long_inter": dict(H=512, I=6656, E=16, G=4, Kg=2, K=4, weight_dtype=DT_MXFP4),
    # 2^20 routed rows x I = 2560: the down GEMM's activations span 5.4 GB, past the
    # 32-bit offsets of the 128-byte-stage GEMM (the 64-byte-stage one, 64-bit addresses)
    "rows_past_4gb": dict(H=256, I=2560, E=64, G=8, Kg=4, K=32),
}


@pytest.mark.parametrize("case,T", [("max_hidden_topk", 16), ("max_hidden_topk", 300), ("single_group", 100),
                                    ("single_group", 700), ("all_groups_kept", 64), ("k1", 50),
                                    ("two_experts", 40), ("short_chunks", 4096), ("short_chunks", 16384),
                                    ("fp8_long_hidden", 300), ("fp8_long_inter", 300), ("mxfp4_long_hidden", 300),
                                    ("mxfp4_long_inter", 300), ("rows_past_4gb", 32768)])
def test_config_limits_and_degenerate_routing(case, T):
    from beam_inputs import Workload, make_inputs
    w = Workload(f"edge_{case}", T=T, seed=3, x_recipe="rms_normal", **_EDGE[case])
    print(f"[case] edge {case} T={T}", flush=True)
    full = make_inputs(w)
    dev = {"w_router": torch.from_numpy(full.w_router).cuda()}
    if w.weight_dtype == DT_BF16:
        dev["w13"] = torch.from_numpy(full.w13.view(np.int16)).cuda().view(torch.bfloat16)
        dev["w2"] = torch.from_numpy(full.w2.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        dev["w13"] = torch.from_numpy(full.w13).cuda()
        dev["w2"] = torch.from_numpy(full.w2).cuda()
    if full.w13_scale is not None:
        dev["w13_scale"] = torch.from_numpy(full.w13_scale).cuda()
        dev["w2_scale"] = torch.from_numpy(full.w2_scale).cuda()
    cfg, y, ids, wts, ws = run_forward(w, dev, full.x, None)
    tok = np.arange(T) if T <= 1000 else sample_tokens(T)
    ref = oracle.moe_forward(x_f32(w, full.x), full.w_router, None, bank_of(w, full), w.G, w.Kg, w.K, w.alpha,
                             token_subset=tok)
    m = bm.beam_moe_workspace_map(cfg, w.T)
    z = ws_region(ws, m["logits"], w.T * w.E, np.float32).reshape(w.T, w.E)
    assert np.array_equal(z, ref["logits"])            # logits bit for bit
    check_routing(w, ids, wts, ref["ids"], ref["w"])
    check_permutation(w, ws, ids)
    if w.K == 1:
        assert (wts == np.float32(w.alpha)).all()
    if w.K == w.E:
        assert (np.sort(ids, axis=1) == np.arange(w.E)).all()
    err = rel_inf(y.float().cpu().numpy()[tok].astype(np.float64), ref["y"])
    print(f"[case] edge {case} T={T} rel_inf={err:.3e}", flush=True)
    assert err <= TOL[w.weight_dtype]
