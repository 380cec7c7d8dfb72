"""Seeded synthetic inputs for the Beam MoE layer.

This module only *makes inputs*: it draws seeded normal tensors, rounds them to
the storage formats the layer consumes (BF16, OCP FP8 E4M3 with block scales)
and builds the skewed logit offsets of the load-imbalanced workload.  It holds
none of the layer's arithmetic (no routing, no expert MLP, no norm), so both the
CPU oracle and the GPU library can consume exactly the same bytes from it.

Random streams: numpy's Philox4x32-10 bit generator (Salmon et al., SC'11,
"Parallel random numbers: as easy as 1, 2, 3"), keyed per tensor and per
expert through a SeedSequence, so any one expert's weights can be regenerated
on its own.  Normal variates come from numpy's `standard_normal` in float32.

Shapes follow the Beam MoE layer (Reflection Beam 1.0 overview, sections
"Architecture" and "Mixture of Experts: 256 experts, 8 routed per token"):
hidden 5120, 256 experts in 8 groups of 32, top-4 groups, top-8 experts,
SwiGLU intermediate 2560, combine scale 2.5.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# Stream tags: one per tensor kind.
TAG_X = 1
TAG_WROUTER = 2
TAG_W13 = 3
TAG_W2 = 4
TAG_PERM = 5
TAG_H = 6
TAG_DW13 = 7      # dense MLP gate/up weights
TAG_DW2 = 8       # dense MLP down weights

DT_F32, DT_BF16, DT_FP8, DT_MXFP4 = 0, 1, 2, 3
DTYPE_NAMES = {DT_F32: "f32", DT_BF16: "bf16", DT_FP8: "fp8_e4m3", DT_MXFP4: "mxfp4"}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def rng(seed: int, *tags: int) -> np.random.Generator:
    """Philox4x32-10 stream keyed by (seed, *tags)."""
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, *tags])))


def normal(seed: int, tags: tuple, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draw of `shape` from the stream keyed by (seed, *tags)."""
    out = np.empty(shape, np.float32)
    rng(seed, *tags).standard_normal(out=out, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns the uint16 bit patterns.

    Inputs are finite by construction (normal draws), so NaN handling is not needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


E4M3_MAX = 448.0


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Encode float32 values (already divided by their scale) as OCP E4M3FN codes.

    Round to nearest even on the E4M3 grid, saturating at +-448 (the format has
    no infinity).  Grid: for |q| >= 2^-6 the step is 2^(floor(log2|q|)-3); below
    that (subnormals) the step is 2^-9.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    # exponent of |v| (frexp: a = m * 2^e, m in [0.5,1)) -> floor(log2 a) = e-1
    _, e = np.frexp(a)
    e = np.maximum(e - 1, -6)
    step = np.ldexp(1.0, e - 3)
    q = np.rint(a / step) * step          # exact in float64; rint is ties-to-even
    q = np.minimum(q, E4M3_MAX)
    # encode the (exactly representable) q
    _, e2 = np.frexp(q)
    e2 = e2 - 1
    normal_ = q >= 2.0 ** -6
    exp_field = np.where(normal_, e2 + 7, 0)
    mant = np.where(normal_, q / np.ldexp(1.0, e2) - 1.0, q / 2.0 ** -9 / 8.0) * 8.0
    mant = np.rint(mant).astype(np.int64)
    code = (exp_field.astype(np.int64) << 3) | mant
    code = np.where(q == 0, 0, code)
    code |= np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


FP8_SCALE_KINDS = ("amax", "pow2")


def quantize_e4m3_blocks(w: np.ndarray, block: int = 128, kind: str = "amax"):
    """Block-scaled E4M3 quantisation of a [N, K] float32 matrix.

    Each block x block tile gets one float32 scale (1 for an all-zero tile):
      "amax": scale = amax / 448 rounded to float32, so the tile's largest magnitude
              maps to the top of the E4M3 range (any float32 value);
      "pow2": the smallest power of two with amax / scale <= 448, so the scale is
              exactly an E8M0 block exponent (amax / scale in (224, 448]).
    codes = E4M3(w / scale), computed in float32 (round to nearest even, saturating
    at 448).  Returns (codes uint8 [N, K], scales float32 [N/block, K/block]).
    """
    assert kind in FP8_SCALE_KINDS, kind
    n, k = w.shape
    assert n % block == 0 and k % block == 0
    t = w.reshape(n // block, block, k // block, block)
    amax = np.abs(t).max(axis=(1, 3)).astype(np.float32)
    if kind == "amax":
        scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    else:
        # ceil(log2(amax / 448)) from the exact binary exponent: frexp gives m in [0.5, 1)
        m, ex = np.frexp(amax.astype(np.float64) / E4M3_MAX)
        ex = np.where(m == 0.5, ex - 1, ex)
        scale = np.where(amax > 0, np.ldexp(1.0, ex), 1.0).astype(np.float32)
    scaled = (t / scale[:, None, :, None]).astype(np.float32)
    codes = encode_e4m3(scaled).reshape(n, k)
    return codes, scale


# MXFP4 (OCP Microscaling Formats (MX) v1.0): blocks of 32 consecutive values along K
# share one E8M0 scale 2^X; the elements are FP4 E2M1 (sign, 2 exponent bits with bias
# 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
MX_BLOCK = 32
E2M1_MAX = 6.0
E2M1_EMAX = 2          # exponent of the largest normal E2M1 value (6 = 1.5 * 2^2)


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Encode values (already divided by their block scale) as E2M1 codes (uint8, low 4
    bits): round to nearest, ties to the even code (mantissa bit 0), saturating at +-6."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    # steps: 0.5 below 2, 1 in [2, 4), 2 in [4, 6]
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.rint(a / step) * step                       # rint: ties to even multiples
    q = np.minimum(q, E2M1_MAX)
    # q is on the grid; code: 0..1 subnormal/zero (0, 0.5), then (e, m)
    _, e = np.frexp(np.where(q > 0, q, 1.0))
    e = e - 1                                          # q = 1.m * 2^e for q >= 1
    exp_field = np.where(q >= 1.0, e + 1, 0)
    mant = np.where(q >= 1.0, q / np.ldexp(1.0, e) - 1.0, q / 0.5) * 2.0
    mant = np.where(q >= 1.0, mant, q / 0.5)
    code = (exp_field.astype(np.int64) << 1) | np.rint(mant).astype(np.int64)
    code = np.where(q == 0, 0, code)
    code |= np.where(np.signbit(v) & (q > 0), 0x8, 0)
    return code.astype(np.uint8)


def quantize_mxfp4(w: np.ndarray):
    """MX quantisation of a [N, K] float32 matrix along K.

    Per block of 32: X = floor(log2(amax)) - 2 (the E2M1 emax), scale 2^X stored as the
    E8M0 code X + 127 (an all-zero block gets code 127), elements E2M1(w / 2^X) with
    round-to-nearest-even and saturation at +-6.  Returns (packed codes uint8 [N, K/2],
    element 2j in the low nibble of byte j; scales uint8 [N, K/32])."""
    n, k = w.shape
    assert k % MX_BLOCK == 0
    t = w.reshape(n, k // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.abs(t).max(axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, (ex - 1) - E2M1_EMAX, 0)
    X = np.clip(X, -127, 127)
    codes = encode_e2m1(t / np.ldexp(1.0, X)[:, :, None]).reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """One synthetic MoE-layer workload: shapes, dtypes and input recipe."""
    name: str
    T: int
    H: int
    I: int
    E: int
    G: int
    Kg: int
    K: int
    alpha: float = 2.5
    act_dtype: int = DT_BF16
    weight_dtype: int = DT_BF16
    x_recipe: str = "normal"      # "normal" | "rms_normal"
    zipf_s: float | None = None    # skewed routing: per-expert logit offsets
    sublayer: bool = False         # pre-norm -> MoE -> post-norm -> residual
    dense: bool = False            # dense SwiGLU MLP (one weight set, no router) in place of the MoE
    step_k: int = 10
    norm_eps: float = 1e-6
    fp8_block: int = 128
    fp8_scales: str = "amax"       # FP8 block scales: "amax" (amax / 448) or "pow2"
    seed: int = 0

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS = {
    # tiny layer, FP32 throughout
    "tiny_f32": Workload("tiny_f32", T=64, H=128, I=64, E=16, G=4, Kg=2, K=4,
                         act_dtype=DT_F32, weight_dtype=DT_F32),
    # Beam-shaped decode batch, BF16 experts, weight streaming
    "beam_decode_t16": Workload("beam_decode_t16", T=16, H=5120, I=2560, E=256, G=8, Kg=4, K=8,
                                x_recipe="rms_normal"),
    # Beam-shaped prefill, near-uniform routing
    "beam_prefill_t4096": Workload("beam_prefill_t4096", T=4096, H=5120, I=2560, E=256, G=8, Kg=4, K=8),
    # Beam-shaped prefill with Zipf(1.1) skewed routing
    "beam_skewed_t32768": Workload("beam_skewed_t32768", T=32768, H=5120, I=2560, E=256, G=8, Kg=4, K=8,
                                   zipf_s=1.1),
    # full sublayer with FP8 experts (block scales amax / 448)
    "beam_sublayer_fp8_t8192": Workload("beam_sublayer_fp8_t8192", T=8192, H=5120, I=2560, E=256, G=8,
                                        Kg=4, K=8, weight_dtype=DT_FP8, sublayer=True),
    # the same with power-of-two block scales (E8M0 block exponents)
    "beam_sublayer_fp8pow2_t8192": Workload("beam_sublayer_fp8pow2_t8192", T=8192, H=5120, I=2560, E=256,
                                            G=8, Kg=4, K=8, weight_dtype=DT_FP8, sublayer=True,
                                            fp8_scales="pow2"),
    # MXFP4 experts (E2M1 elements, E8M0 scale per 32 along K): decode batch and prefill
    "beam_decode_mxfp4_t16": Workload("beam_decode_mxfp4_t16", T=16, H=5120, I=2560, E=256, G=8, Kg=4, K=8,
                                      weight_dtype=DT_MXFP4, x_recipe="rms_normal"),
    "beam_prefill_mxfp4_t4096": Workload("beam_prefill_mxfp4_t4096", T=4096, H=5120, I=2560, E=256, G=8, Kg=4,
                                         K=8, weight_dtype=DT_MXFP4),
    # dense SwiGLU MLP of the first decoder layers, width 8 x 2560 = 20480 (the routed
    # width of one MoE layer; the pages do not give the dense width)
    "beam_dense_decode_t16": Workload("beam_dense_decode_t16", T=16, H=5120, I=20480, E=1, G=1, Kg=1, K=1,
                                      alpha=1.0, dense=True, x_recipe="rms_normal"),
    "beam_dense_prefill_t4096": Workload("beam_dense_prefill_t4096", T=4096, H=5120, I=20480, E=1, G=1, Kg=1,
                                         K=1, alpha=1.0, dense=True),
}


def zipf_logit_offsets(E: int, s: float, seed: int) -> np.ndarray:
    """Per-expert logit offsets b_e = ln(E * p_{r(e)}), p_r = r^-s / sum_j j^-s.

    r(e) is expert e's rank (1-based) under a seeded random permutation of the
    experts, so a few experts receive many times the mean load.
    """
    perm = rng(seed, TAG_PERM).permutation(E)
    rank = np.empty(E, np.int64)
    rank[perm] = np.arange(1, E + 1)
    j = np.arange(1, E + 1, dtype=np.float64)
    p = rank.astype(np.float64) ** (-s) / np.sum(j ** (-s))
    return np.log(E * p).astype(np.float32)


def token_inputs(w: Workload) -> np.ndarray:
    """Activations [T, H] as float32 (values already on the storage grid).

    "normal": i.i.d. N(0,1); "rms_normal": each row divided by its RMS.
    For the sublayer workload this is the residual stream h ~ N(0,1).
    Rows are drawn one 16-row chunk at a time so a prefix of rows does not
    depend on T.
    """
    tag = TAG_H if w.sublayer else TAG_X
    chunks = []
    for c0 in range(0, w.T, 16):
        n = min(16, w.T - c0)
        z = normal(w.seed, (tag, c0 // 16), (16, w.H))[:n]
        chunks.append(z)
    z = np.concatenate(chunks, axis=0) if chunks else np.zeros((0, w.H), np.float32)
    if w.x_recipe == "rms_normal":
        rms = np.sqrt(np.mean(z.astype(np.float64) ** 2, axis=1, keepdims=True))
        z = (z / rms).astype(np.float32)
    return z


@dataclass
class Inputs:
    """Materialised inputs of one workload (host memory, storage formats)."""
    w: Workload
    x: np.ndarray                  # [T,H] float32 (F32 acts) or uint16 BF16 bits
    w_router: np.ndarray | None    # [H,E] float32 (None for the dense MLP)
    logit_bias: np.ndarray | None  # [E] float32 or None
    w13: np.ndarray                # [E,2I,H] float32 | uint16 bf16 bits | uint8 e4m3
    w2: np.ndarray                 # [E,H,I]  same dtype family as w13
    w13_scale: np.ndarray | None = None   # [E,2I/128,H/128] float32 (FP8 only)
    w2_scale: np.ndarray | None = None    # [E,H/128,I/128]  float32 (FP8 only)
    extra: dict = field(default_factory=dict)


def _expert_draw(w: Workload, e: int):
    t13, t2 = (TAG_DW13, TAG_DW2) if w.dense else (TAG_W13, TAG_W2)
    g13 = normal(w.seed, (t13, e), (2 * w.I, w.H), std=1.0 / math.sqrt(w.H))
    g2 = normal(w.seed, (t2, e), (w.H, w.I), std=1.0 / math.sqrt(w.I))
    return g13, g2


def make_inputs(w: Workload, experts: list[int] | None = None) -> Inputs:
    """Generate all inputs of workload `w`.

    Weights are N(0, std = 1/sqrt(fan_in)); fan_in = H for the router, gate and up
    projections, I for the down projection.  If `experts` is given, only those
    experts' weight slots are filled (the rest stay zero) - used to keep CPU-side
    checks small at Beam size.
    """
    x = token_inputs(w)
    if w.act_dtype == DT_BF16:
        x = to_bf16_bits(x)
    # the dense MLP has no router: its single weight set is slot 0 of w13 / w2
    w_router = None if w.dense else normal(w.seed, (TAG_WROUTER,), (w.H, w.E), std=1.0 / math.sqrt(w.H))
    bias = zipf_logit_offsets(w.E, w.zipf_s, w.seed) if w.zipf_s is not None else None
    E, I, H = w.E, w.I, w.H
    if w.weight_dtype == DT_F32:
        w13 = np.zeros((E, 2 * I, H), np.float32)
        w2 = np.zeros((E, H, I), np.float32)
    elif w.weight_dtype == DT_BF16:
        w13 = np.zeros((E, 2 * I, H), np.uint16)
        w2 = np.zeros((E, H, I), np.uint16)
    elif w.weight_dtype == DT_FP8:
        w13 = np.zeros((E, 2 * I, H), np.uint8)
        w2 = np.zeros((E, H, I), np.uint8)
    else:
        w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
        w2 = np.zeros((E, H, I // 2), np.uint8)
    s13 = s2 = None
    if w.weight_dtype == DT_FP8:
        b = w.fp8_block
        s13 = np.ones((E, 2 * I // b, H // b), np.float32)
        s2 = np.ones((E, H // b, I // b), np.float32)
    elif w.weight_dtype == DT_MXFP4:
        s13 = np.full((E, 2 * I, H // MX_BLOCK), 127, np.uint8)
        s2 = np.full((E, H, I // MX_BLOCK), 127, np.uint8)

    todo = list(range(E)) if experts is None else sorted(set(experts))

    def fill(e):
        g13, g2 = _expert_draw(w, e)
        if w.weight_dtype == DT_F32:
            w13[e], w2[e] = g13, g2
        elif w.weight_dtype == DT_BF16:
            w13[e], w2[e] = to_bf16_bits(g13), to_bf16_bits(g2)
        elif w.weight_dtype == DT_FP8:
            w13[e], s13[e] = quantize_e4m3_blocks(g13, w.fp8_block, w.fp8_scales)
            w2[e], s2[e] = quantize_e4m3_blocks(g2, w.fp8_block, w.fp8_scales)
        else:
            w13[e], s13[e] = quantize_mxfp4(g13)
            w2[e], s2[e] = quantize_mxfp4(g2)

    if len(todo) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, todo))
    else:
        for e in todo:
            fill(e)
    return Inputs(w, x, w_router, bias, w13, w2, s13, s2)
