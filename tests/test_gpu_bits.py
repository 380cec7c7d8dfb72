"""Bit-for-bit pins of the GPU's FP32 router arithmetic against the CPU oracle, through
the C ABI (the routing contract in beam_moe.h: the scores s = 1 / (1 + exp(-z)) with the
own Cody-Waite exponential and an IEEE division; the pre-norm's correctly rounded
square root and division; Reflection Beam 1.0 overview, "Residual stream": the router and
the norms run in FP32).

Sigmoid: every FP32 bit pattern z with |z| <= 87 (about 2.2e9 values) is routed as a
logit.  A token whose activations are one-hot at hidden index h has logits z[e] =
W_r[h, e] exactly under the 64-chunk order (one fused multiply-add by 1 into a zero
accumulator, every other product a signed zero; a weight of -0 gives +0), so a router
weight matrix filled with consecutive bit patterns and the identity as activations route
every pattern once; the scores region of the workspace is compared with the oracle's
sigmoid bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_group_amd as bm

pytestmark = pytest.mark.gpu

H, E = 16384, 256          # the largest hidden size the kernels take; 256 experts
Z_MAX_BITS = 0x42AE0000    # 87.0f


def _ws_region(ws, off, count, dtype):
    return ws[off:off + count * np.dtype(dtype).itemsize].cpu().numpy().view(dtype)


def test_router_sigmoid_every_fp32_in_clamp_range():
    cfg = bm.make_config(hidden=H, inter=128, n_experts=E, n_groups=8, topk_groups=4, topk=8)
    T = H
    x = torch.eye(T, H, dtype=torch.bfloat16, device="cuda")        # token t one-hot at h = t
    ws = bm.alloc_workspace(cfg, T)
    m = bm.beam_moe_workspace_map(cfg, T)
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    n = H * E
    total = 0
    for sign in (0, 0x80000000):
        for start in range(0, Z_MAX_BITS + 1, n):
            cnt = min(n, Z_MAX_BITS + 1 - start)
            bits = np.arange(start, start + n, dtype=np.uint32)
            bits[cnt:] = start                          # pad the last batch with its first value
            bits |= np.uint32(sign)
            zf = bits.view(np.float32)
            wr = torch.from_numpy(zf.reshape(H, E)).cuda()
            bm.beam_moe_route(cfg, x, wr, ids=ids, weights=wts, ws=ws)
            torch.cuda.synchronize()
            z_gpu = _ws_region(ws, m["logits"], T * E, np.float32)
            s_gpu = _ws_region(ws, m["scores"], T * E, np.float32)
            # the weight itself, except that -0 comes out +0 (a zero accumulator plus -0)
            z_ref = np.where(bits == np.uint32(0x80000000), np.uint32(0), bits)
            assert np.array_equal(z_gpu.view(np.uint32), z_ref), "one-hot logits are not the weights"
            s_ref = oracle.sigmoidf(zf)
            bad = np.flatnonzero(s_gpu.view(np.uint32) != s_ref.view(np.uint32))
            assert bad.size == 0, (f"{bad.size} scores differ, first z={zf[bad[0]]!r} "
                                   f"gpu={s_gpu[bad[0]]!r} cpu={s_ref[bad[0]]!r}")
            total += cnt
        print(f"[case] sigmoid bits sign={sign:#x} checked through {start + cnt:#x}", flush=True)
    assert total == 2 * (Z_MAX_BITS + 1)


def test_prenorm_bits_over_many_mean_squares():
    """The sublayer's FP32 pre-norm (sum of squares in the fixed order, correctly rounded
    division and square root, xhat = (h * r) * g) against the oracle's, bit for bit, on
    rows whose mean squares span 2^-40 .. 2^40: constant rows, one-hot rows and Gaussian
    rows scaled by powers of two, with a non-unit gain."""
    Hs = 1024
    cfg = bm.make_config(hidden=Hs, inter=128, n_experts=16, n_groups=4, topk_groups=2, topk=4)
    rs = np.random.default_rng(12)
    rows = []
    for e in range(-20, 21):
        c = np.float32(2.0 ** e * (1 + rs.random()))
        rows.append(np.full(Hs, c, np.float32))                      # constant row
        one = np.zeros(Hs, np.float32); one[rs.integers(Hs)] = c
        rows.append(one)                                              # one nonzero entry
        rows.append((rs.standard_normal(Hs) * 2.0 ** e).astype(np.float32))
    from beam_inputs import to_bf16_bits
    hb = to_bf16_bits(np.stack(rows))
    T = hb.shape[0]
    gain = (1 + 0.25 * rs.standard_normal(Hs)).astype(np.float32)
    h = torch.from_numpy(hb.view(np.int16)).cuda().view(torch.bfloat16)
    w13 = torch.zeros((16, 256, Hs), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((16, Hs, 128), dtype=torch.bfloat16, device="cuda")
    wr = torch.from_numpy((rs.standard_normal((Hs, 16)) / 32).astype(np.float32)).cuda()
    ws = bm.alloc_workspace(cfg, T)
    bm.beam_moe_sublayer_forward(cfg, h, 10, wr, w13, w2, pre_gain=torch.from_numpy(gain).cuda(), ws=ws)
    torch.cuda.synchronize()
    m = bm.beam_moe_workspace_map(cfg, T)
    xg = _ws_region(ws, m["xhat"], T * Hs, np.float32).reshape(T, Hs)
    xr, _ = oracle.prenorm(oracle.bf16_to_f32(hb), gain, 1e-6)
    bad = np.argwhere(xg.view(np.uint32) != xr.view(np.uint32))
    if bad.size:
        t, c = bad[0]
        print(f"[case] prenorm bits: {len(bad)} differ in rows {np.unique(bad[:, 0])[:12]}; first row {t} col {c}: "
              f"gpu={xg[t, c]!r} cpu={xr[t, c]!r} h={oracle.bf16_to_f32(hb)[t, c]!r}", flush=True)
    assert bad.size == 0
