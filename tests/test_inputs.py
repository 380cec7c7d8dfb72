"""Checks of the seeded input generator (beam_inputs) against independent routines."""
import math
import numpy as np
import torch

import oracle
from beam_inputs import (DT_F32, WORKLOADS, encode_e4m3, encode_e2m1, make_inputs, quantize_e4m3_blocks, quantize_mxfp4,
                         to_bf16_bits,
                         token_inputs, zipf_logit_offsets, normal)


def test_bf16_rounding_matches_torch():
    rs = np.random.default_rng(0)
    a = (rs.standard_normal(1_000_000) * np.exp(rs.uniform(-20, 20, 1_000_000))).astype(np.float32)
    mine = to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_e4m3_encoding_matches_torch_rne_saturating():
    rs = np.random.default_rng(1)
    v = (rs.standard_normal(500_000) * np.exp(rs.uniform(-8, 6, 500_000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    mine = encode_e4m3(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    # every finite code round-trips
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_to_f64(codes).astype(np.float32)
    rt = encode_e4m3(vals)
    assert np.array_equal(oracle.e4m3_to_f64(rt), oracle.e4m3_to_f64(codes))


def test_block_quantisation_amax_scales():
    """amax / 448 block scales (the plain reading of FP32 block scales): each tile's
    largest magnitude maps onto the E4M3 maximum, 448, and the stored values are within
    half an E4M3 step of the weights."""
    w = normal(0, (5,), (256, 384), std=0.02)
    w[128:, 256:] = 0.0                                   # an all-zero block
    codes, scales = quantize_e4m3_blocks(w, 128, "amax")
    assert scales.shape == (2, 3) and scales.dtype == np.float32
    assert scales[1, 2] == 1.0
    deq = oracle.dequant_blocks(codes, scales, 128)
    m, _ = np.frexp(scales[:1].astype(np.float64))
    assert not np.all(m == 0.5)                           # not merely powers of two
    for i in range(2):
        for j in range(3):
            if i == 1 and j == 2:
                continue
            t = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            amax = np.abs(t).max()
            assert scales[i, j] == np.float32(amax) / np.float32(448.0)
            c = codes[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert (np.abs(oracle.e4m3_to_f64(c)) == 448.0).any()        # the amax element
            d = deq[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            # |w| / scale in a binade [2^e, 2^(e+1)) has step 2^(e-3): error <= step / 2
            q = np.abs(t).astype(np.float64) / float(scales[i, j])
            e = np.floor(np.log2(np.maximum(q, 2.0 ** -6))).astype(np.int64)
            step = np.ldexp(1.0, e - 3)
            assert np.all(np.abs(d - t) <= step / 2 * scales[i, j] * (1 + 1e-6) + 1e-12)
    assert np.all(deq[128:, 256:] == 0.0)


def test_block_quantisation_power_of_two_scales():
    w = normal(0, (5,), (256, 384), std=0.02)
    w[128:, 256:] = 0.0                                   # an all-zero block
    codes, scales = quantize_e4m3_blocks(w, 128, "pow2")
    assert scales.shape == (2, 3)
    m, _ = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)                               # exact powers of two (E8M0)
    assert scales[1, 2] == 1.0
    deq = oracle.dequant_blocks(codes, scales, 128)
    for i in range(2):
        for j in range(3):
            if i == 1 and j == 2:
                continue
            blk = np.abs(w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]).max()
            assert 224.0 < blk / scales[i, j] <= 448.0    # smallest such power of two
    assert np.all(deq[128:, 256:] == 0.0)
    rel = np.abs(deq - w) / np.abs(w).max()
    assert rel.max() <= 2.0 ** -4 + 1e-6      # half a step of a 3-bit mantissa at amax


def test_e2m1_encoder_round_to_nearest_even_and_saturation():
    grid = oracle.E2M1_TABLE[:8]
    # every representable value round-trips; midpoints go to the even code
    assert np.array_equal(oracle.E2M1_TABLE[encode_e2m1(grid)], grid)
    assert np.array_equal(oracle.E2M1_TABLE[encode_e2m1(-grid[1:])], -grid[1:])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert np.array_equal(oracle.E2M1_TABLE[encode_e2m1(mids)], [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    assert np.array_equal(oracle.E2M1_TABLE[encode_e2m1(np.array([6.5, 100.0, -7.0]))], [6.0, 6.0, -6.0])
    # off-midpoint values go to the nearest grid point
    v = np.random.default_rng(3).uniform(-6, 6, 20000)
    got = oracle.E2M1_TABLE[encode_e2m1(v)]
    dist = np.abs(v[:, None] - np.concatenate([grid, -grid])[None, :]).min(axis=1)
    assert np.allclose(np.abs(got - v), dist)


def test_mxfp4_block_scales_follow_the_mx_rule():
    """X = floor(log2(amax)) - 2 per block of 32 along K (OCP MX v1.0 conversion with the
    E2M1 emax of 2); amax / 2^X lies in [4, 8), so the block maximum rounds to 4 or 6."""
    w = normal(0, (9,), (64, 256), std=0.02)
    w[3, 32:64] = 0.0
    packed, sc = quantize_mxfp4(w)
    assert packed.shape == (64, 128) and sc.shape == (64, 8)
    amax = np.abs(w.reshape(64, 8, 32)).max(axis=2).astype(np.float64)
    X = sc.astype(np.int64) - 127
    nz = amax > 0
    assert np.array_equal(X[nz], np.floor(np.log2(amax[nz])).astype(np.int64) - 2)
    assert sc[3, 1] == 127
    deq = oracle.dequant_mxfp4(packed, sc)
    assert np.all(deq[3, 32:64] == 0.0)
    # elements up to 6 * 2^X lie within half a grid step (at most 2^X at the top, where
    # the step is 2 * 2^X); larger ones saturate to 6 * 2^X (amax / 2^X < 8)
    scale = np.repeat(np.ldexp(1.0, X), 32, axis=1)
    err = np.abs(deq - w)
    inside = np.abs(w) <= 6.0 * scale
    assert np.all(err[inside] <= scale[inside] + 1e-12)
    assert np.all(deq[~inside] == np.sign(w[~inside]) * 6.0 * scale[~inside])
    assert np.all(err < 2.0 * scale)


def test_prefix_rows_independent_of_T():
    w = WORKLOADS["beam_prefill_t4096"]
    a = token_inputs(w.with_T(16))
    b = token_inputs(w.with_T(40))
    assert np.array_equal(a, b[:16])


def test_zipf_offsets_skew():
    b = zipf_logit_offsets(256, 1.1, 0)
    p = np.exp(b.astype(np.float64)) / 256
    assert abs(p.sum() - 1) < 1e-5
    assert b.max() > 3.9 and b.min() < -2.0


def test_tiny_inputs_shapes():
    inp = make_inputs(WORKLOADS["tiny_f32"])
    assert inp.x.shape == (64, 128) and inp.x.dtype == np.float32
    assert inp.w13.shape == (16, 128, 128) and inp.w2.shape == (16, 128, 64)


def test_dense_workload_draws_its_own_weights():
    """The dense MLP has no router and one weight set, drawn from its own streams (not
    expert 0's); the fan-in scaling is the experts' (1/sqrt(H), 1/sqrt(I))."""
    from dataclasses import replace
    d = replace(WORKLOADS["beam_dense_decode_t16"], H=256, I=512, T=4, weight_dtype=DT_F32, act_dtype=DT_F32)
    inp = make_inputs(d)
    assert inp.w_router is None and inp.w13.shape == (1, 1024, 256) and inp.w2.shape == (1, 256, 512)
    moe = make_inputs(replace(d, dense=False, E=2, G=1, Kg=1, K=1), experts=[0])
    assert not np.array_equal(inp.w13[0], moe.w13[0])
    assert abs(inp.w13.std() * 16 - 1) < 0.02 and abs(inp.w2.std() * math.sqrt(512) - 1) < 0.02


def test_e4m3_activation_error_barely_depends_on_scale_granularity():
    """Why the GPU quantises activations with one scale per row: E4M3 keeps 3 mantissa
    bits whatever the scale, so as long as a row's values stay in the normal range the
    relative rounding error (and the error of a dot product over 5120 terms) is the same
    for one scale per row, per 1 x 128 block or per 32 values.  Measured on RMS-normalised
    Gaussian rows and N(0, 1/H) weights: every granularity within 10% of the per-row one."""
    rs = np.random.default_rng(0)
    T, H, N = 32, 5120, 256
    x = rs.standard_normal((T, H)).astype(np.float32)
    x /= np.sqrt((x.astype(np.float64) ** 2).mean(1, keepdims=True)).astype(np.float32)
    w = (rs.standard_normal((N, H)) / np.sqrt(H)).astype(np.float32)
    ref = x.astype(np.float64) @ w.T.astype(np.float64)

    def quant(block):
        xb = x.reshape(T, H // block, block)
        s = (np.abs(xb).max(axis=2, keepdims=True) / np.float32(448.0)).astype(np.float32)
        q = oracle.e4m3_to_f64(encode_e4m3((xb / s).astype(np.float32)))
        return (q * s).reshape(T, H)

    errs = {}
    for name, block in (("row", H), ("1x128", 128), ("1x32", 32)):
        y = quant(block) @ w.T.astype(np.float64)
        errs[name] = float(np.sqrt(((y - ref) ** 2).mean() / (ref ** 2).mean()))
    assert 0.015 < errs["row"] < 0.035, errs
    for name in ("1x128", "1x32"):
        assert abs(errs[name] / errs["row"] - 1) < 0.10, errs
