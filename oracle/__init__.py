"""CPU oracle for the Beam MoE layer -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and `bench.py`'s CPU-baseline leg may
import this package.  It shares no code with the GPU library
(`sparse_mixture_experts_group_amd`) and never imports it; the only module both
use is `beam_inputs`, which makes the seeded input bytes.

What the layer computes (Reflection Beam 1.0 overview, section "Mixture of
Experts: 256 experts, 8 routed per token"; the residual and norm sublayer from
section "Residual stream: depth-dependent weights keep the hidden state at
constant scale"):

  router   z = x . Wr (+ b);  s = sigmoid(z)                        FP32 (C)
  groups   score_g = top1 + top2 of s inside group g; keep Kg       FP32 (C)
  experts  top-K of s inside the kept groups; w_i = alpha s_i / sum  FP32 (C)
  experts  a = SiLU(x Wg^T) * (x Wu^T);  o = a Wd^T                  float64
  combine  y = sum_i w_i o_i                                          float64
  sublayer h' = sqrt((k-1)/k) h + (1/sqrt k) RMSNorm(y),
           with the MoE input RMSNorm(h) (FP32, C)                    float64
  dense    y = Wd (SiLU(Wg x) * (Wu x)), the MLP of the first 3 layers
           (section "Architecture"), alone or inside the same sublayer float64

The router and the pre-norm are FP32 because the pages fix those sites to FP32
and their result decides integers (expert ids); every other step is float64, a
tighter reference than the FP32 floor the pages set.

Optional operand model for 8-bit expert weights (`ExpertBank(act_quant=True)`): the
GEMMs' activation operands as E4M3 rows with an FP32 amax/448 scale, x as given and the
SwiGLU output after FP32 and BF16 rounding (`quant_rows_e4m3`, `bf16_round`); products
and sums stay float64.  The pages name FP8 checkpoints but not the activation format,
so this is a reading; tests compare the GPU against the oracle with and without it.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "beam_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libbeam_oracle.so")
GCC_FLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-mfma", "-mavx2", "-Wall"]


def build() -> str:
    """Compile oracle/beam_oracle.c into oracle/libbeam_oracle.so (gcc)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        f32p = ctypes.POINTER(ctypes.c_float)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64 = ctypes.c_int64
        L.oracle_expf.restype = ctypes.c_float
        L.oracle_expf.argtypes = [ctypes.c_float]
        L.oracle_sigmoidf.restype = ctypes.c_float
        L.oracle_sigmoidf.argtypes = [ctypes.c_float]
        L.oracle_expf_array.argtypes = [i64, f32p, f32p]
        L.oracle_sigmoidf_array.argtypes = [i64, f32p, f32p]
        L.oracle_router_logits.argtypes = [i64, ctypes.c_int, ctypes.c_int, f32p, f32p, f32p, f32p]
        L.oracle_route.argtypes = [i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_float, f32p, f32p, i32p, f32p, f32p, f32p, i32p]
        L.oracle_prenorm.argtypes = [i64, ctypes.c_int, f32p, f32p, ctypes.c_float, f32p, f32p]
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _f32p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _i32p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ---------------------------------------------------------------------------
# storage-format decoding (the oracle's own; never shared with the GPU side)
# ---------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly (bf16 = upper half of an fp32)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 OCP FP8 E4M3FN codes (OCP 8-bit Floating Point
    Specification v1.0): sign bit, 4-bit exponent (bias 7), 3-bit mantissa;
    exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinity."""
    tab = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        ex = (c >> 3) & 0xF
        m = c & 0x7
        if ex == 0xF and m == 0x7:
            tab[c] = np.nan
        elif ex == 0:
            tab[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            tab[c] = sign * (1.0 + m / 8.0) * 2.0 ** (ex - 7)
    return tab


E4M3_TABLE = _e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, np.uint8)]


def e4m3_encode(v32: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3FN code of each FP32 value, ties to the even code (the one whose
    mantissa field is even), magnitudes at or past 448 saturated to 448; the sign bit is
    the value's (so -0 -> 0x80).  Written as a search over the 127 non-negative finite
    code values (ascending in code order) to stay obviously correct."""
    v = np.asarray(v32, np.float32)
    a = np.abs(v.astype(np.float64))
    pos = E4M3_TABLE[:0x7F]
    hi = np.clip(np.searchsorted(pos, a, side="left"), 1, 0x7E)
    lo = hi - 1
    d_lo, d_hi = a - pos[lo], pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= 448.0, 0x7E, code)
    code = np.where(a == 0.0, 0, code).astype(np.uint8)
    return code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))


def bf16_round(v32: np.ndarray) -> np.ndarray:
    """FP32 -> bfloat16 by round to nearest even, returned widened to FP32 (finite
    inputs)."""
    b = np.asarray(v32, np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return bf16_to_f32(r.astype(np.uint16))


def quant_rows_e4m3(v32: np.ndarray):
    """E4M3 activation operand of the 8-bit expert GEMMs, one FP32 scale per row: s =
    amax(|row|) / 448 (1 for an all-zero row), codes = E4M3(v * (1/s)) with 1/s and the
    product rounded to FP32 -- the FP32 steps, in this order, decide the codes, so they
    are spelled out.  Returns (codes [R, C] uint8, s [R] float32).  The pages name FP8
    checkpoints (Reflection Beam 1.0 overview, "Key specifications at a glance") but not
    the activations' format; E4M3 rows with an amax scale is the plainest reading."""
    v = np.ascontiguousarray(v32, np.float32)
    amax = np.abs(v).max(axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    return e4m3_encode((v * inv[:, None]).astype(np.float32)), s


def act_e4m3(v32: np.ndarray) -> np.ndarray:
    """Value the 8-bit GEMMs see for FP32 activation rows: code value * row scale
    (float64, exact)."""
    codes, s = quant_rows_e4m3(v32)
    return e4m3_to_f64(codes) * s.astype(np.float64)[:, None]


def dequant_blocks(codes: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """Stored value of a block-scaled E4M3 matrix: code value * its tile's FP32 scale
    (exact in float64)."""
    v = e4m3_to_f64(codes)
    n, k = v.shape
    return (v.reshape(n // block, block, k // block, block)
            * scales.astype(np.float64)[:, None, :, None]).reshape(n, k)


def _e2m1_table() -> np.ndarray:
    """Value of each of the 16 FP4 E2M1 codes (OCP Microscaling Formats v1.0, element
    format FP4): sign bit, 2-bit exponent (bias 1), 1-bit mantissa; exponent field 0
    encodes the subnormal m/2 * 2^0; no infinity or NaN."""
    tab = np.empty(16, np.float64)
    for c in range(16):
        sign = -1.0 if c & 0x8 else 1.0
        ex = (c >> 1) & 0x3
        m = c & 0x1
        tab[c] = sign * ((m / 2.0) if ex == 0 else (1.0 + m / 2.0) * 2.0 ** (ex - 1))
    return tab


E2M1_TABLE = _e2m1_table()


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale (OCP MX v1.0): 2^(code - 127); code 255 is NaN."""
    c = np.asarray(codes, np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """Stored value of an MXFP4 matrix [N, K]: packed [N, K/2] bytes (element 2j in the
    low nibble of byte j, 2j+1 in the high nibble), scales [N, K/block] E8M0; value =
    E2M1 element * its block's scale (exact in float64)."""
    p = np.asarray(packed, np.uint8)
    n, kh = p.shape
    codes = np.empty((n, 2 * kh), np.uint8)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    v = E2M1_TABLE[codes]
    return (v.reshape(n, -1, block) * e8m0_to_f64(scales)[:, :, None]).reshape(n, 2 * kh)


# ---------------------------------------------------------------------------
# FP32 router (C)
# ---------------------------------------------------------------------------
def expf(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty_like(x)
    lib().oracle_expf_array(x.size, _f32p(x), _f32p(y))
    return y


def sigmoidf(z: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, np.float32)
    s = np.empty_like(z)
    lib().oracle_sigmoidf_array(z.size, _f32p(z), _f32p(s))
    return s


def router_logits(x32: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None = None):
    """z [T,E] FP32: 64 contiguous chunks of h, each one ascending fused multiply-add
    chain; chunk sums added in ascending order; then + b[e]."""
    x32 = np.ascontiguousarray(x32, np.float32)
    wr = np.ascontiguousarray(w_router, np.float32)
    T, H = x32.shape
    H2, E = wr.shape
    assert H == H2 and H % 64 == 0
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    z = np.empty((T, E), np.float32)
    lib().oracle_router_logits(T, H, E, _f32p(x32), _f32p(wr), _f32p(b), _f32p(z))
    return z


def route(z: np.ndarray, G: int, Kg: int, K: int, alpha: float, details: bool = False,
          select_bias: np.ndarray | None = None):
    """Group-limited top-K of sigmoid scores.  Returns ids [T,K] int32 (ranking value
    descending, ties to the lower index) and weights [T,K] FP32 (sum = alpha).  With a
    select_bias [E], groups and experts are ranked by s + b (FP32) while the weights
    normalise the unbiased scores s (auxiliary-loss-free balancing bias)."""
    z = np.ascontiguousarray(z, np.float32)
    T, E = z.shape
    assert E % G == 0 and E // G >= 2 and 1 <= Kg <= G and 1 <= K <= Kg * (E // G)
    sb = None if select_bias is None else np.ascontiguousarray(select_bias, np.float32)
    assert sb is None or sb.shape == (E,)
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    s = np.empty((T, E), np.float32) if details else None
    gs = np.empty((T, G), np.float32) if details else None
    gk = np.empty((T, Kg), np.int32) if details else None
    lib().oracle_route(T, E, G, Kg, K, float(alpha), _f32p(z), _f32p(sb), _i32p(ids), _f32p(w),
                       _f32p(s), _f32p(gs), _i32p(gk))
    if details:
        return ids, w, {"scores": s, "group_scores": gs, "kept_groups": gk}
    return ids, w


def prenorm(h32: np.ndarray, gain: np.ndarray | None, eps: float):
    """FP32 RMSNorm with the fixed summation order; returns (xhat [T,H], rstd [T])."""
    h32 = np.ascontiguousarray(h32, np.float32)
    T, H = h32.shape
    g = None if gain is None else np.ascontiguousarray(gain, np.float32)
    out = np.empty_like(h32)
    r = np.empty(T, np.float32)
    lib().oracle_prenorm(T, H, _f32p(h32), _f32p(g), float(eps), _f32p(out), _f32p(r))
    return out, r


# ---------------------------------------------------------------------------
# expert MLPs, combine, post-norm, residual (float64)
# ---------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) (float64)."""
    return g / (1.0 + np.exp(-g))


def expert_gate_up(xrows: np.ndarray, w13: np.ndarray, act_quant: bool = False) -> np.ndarray:
    """SwiGLU hidden rows a = SiLU(x Wg^T) * (x Wu^T) (float64); w13 [2I,H]: gate rows
    0..I-1, up rows I..2I-1.  act_quant: x (FP32 values) enters as E4M3 rows
    (`quant_rows_e4m3`), as the 8-bit GEMMs take it."""
    I = w13.shape[0] // 2
    if act_quant:
        xrows = act_e4m3(np.asarray(xrows).astype(np.float32))
    g = xrows @ w13[:I].T
    u = xrows @ w13[I:].T
    return silu(g) * u


def expert_down(a: np.ndarray, w2: np.ndarray, act_quant: bool = False) -> np.ndarray:
    """Expert output o = a Wd^T (float64); w2 [H,I].  act_quant: a is rounded to FP32,
    stored as BF16 and enters as E4M3 rows, as the 8-bit down GEMM takes it."""
    if act_quant:
        a = act_e4m3(bf16_round(np.asarray(a).astype(np.float32)))
    return a @ w2.T


def expert_ffn(xrows: np.ndarray, w13: np.ndarray, w2: np.ndarray, act_quant: bool = False) -> np.ndarray:
    """SwiGLU expert on rows [n,H] (float64): o = (SiLU(x Wg^T) * (x Wu^T)) Wd^T; with
    act_quant both GEMMs see the E4M3 operands the library forms; products and sums stay
    float64."""
    return expert_down(expert_gate_up(xrows, w13, act_quant), w2, act_quant)


class ExpertBank:
    """Float64 view of stored expert weights, decoded one expert at a time."""

    def __init__(self, w13, w2, dtype: str, w13_scale=None, w2_scale=None, block: int = 128,
                 act_quant: bool = False):
        self.w13, self.w2, self.dtype = w13, w2, dtype
        self.s13, self.s2, self.block = w13_scale, w2_scale, block
        self.act_quant = act_quant          # E4M3 activation operands (expert_ffn)

    def expert(self, e: int):
        if self.dtype == "f32":
            return self.w13[e].astype(np.float64), self.w2[e].astype(np.float64)
        if self.dtype == "bf16":
            return (bf16_to_f32(self.w13[e]).astype(np.float64),
                    bf16_to_f32(self.w2[e]).astype(np.float64))
        if self.dtype == "fp8_e4m3":
            return (dequant_blocks(self.w13[e], self.s13[e], self.block),
                    dequant_blocks(self.w2[e], self.s2[e], self.block))
        if self.dtype == "mxfp4":
            return dequant_mxfp4(self.w13[e], self.s13[e]), dequant_mxfp4(self.w2[e], self.s2[e])
        raise ValueError(self.dtype)


def moe_combine(x64: np.ndarray, ids: np.ndarray, w: np.ndarray, bank: ExpertBank,
                return_expert_outputs: bool = False):
    """y[t] = sum_{i=0..K-1} w[t,i] * FFN_{ids[t,i]}(x[t]) in float64.

    Loops expert by expert (each expert's rows at once) -- the per-token definition
    is unchanged; the loop order only keeps one expert's weights decoded at a time.
    The sum over i is taken in ascending i.
    """
    T, K = ids.shape
    H = x64.shape[1]
    outs = np.zeros((T, K, H), np.float64)
    for e in np.unique(ids):
        t_idx, k_idx = np.nonzero(ids == e)
        w13, w2 = bank.expert(int(e))
        outs[t_idx, k_idx] = expert_ffn(x64[t_idx], w13, w2, bank.act_quant)
    y = combine_outputs(outs, w)
    if return_expert_outputs:
        return y, outs
    return y


def combine_outputs(outs: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[t] = sum_i w[t,i] * outs[t,i] (float64), the sum taken in ascending i."""
    y = np.zeros((outs.shape[0], outs.shape[2]), np.float64)
    for i in range(outs.shape[1]):
        y += w[:, i:i + 1].astype(np.float64) * outs[:, i]
    return y


def rmsnorm64(y: np.ndarray, gain: np.ndarray | None, eps: float) -> np.ndarray:
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + eps)
    out = y * r
    if gain is not None:
        out = out * gain.astype(np.float64)
    return out


def residual_coeffs(k: int):
    """Constant-scale residual at step k: keep sqrt((k-1)/k) of the stream, add
    1/sqrt(k) of the sublayer output (Reflection Beam 1.0 overview, "Residual stream")."""
    return math.sqrt((k - 1) / k), 1.0 / math.sqrt(k)


def residual_update(h64: np.ndarray, out64: np.ndarray, k: int) -> np.ndarray:
    c1, c2 = residual_coeffs(k)
    return c1 * h64 + c2 * out64


def sublayer_output(h32_rows: np.ndarray, y: np.ndarray, post_gain, step_k: int, eps: float) -> np.ndarray:
    """The stream after a sublayer whose output (before the post-norm) is y: the
    post-RMSNorm of y, added with the constant-scale residual weights at step k."""
    return residual_update(h32_rows.astype(np.float64), rmsnorm64(y, post_gain, eps), step_k)


# ---------------------------------------------------------------------------
# whole layer / sublayer
# ---------------------------------------------------------------------------
def moe_forward(x32: np.ndarray, w_router, bias, bank: ExpertBank, G, Kg, K, alpha,
                token_subset: np.ndarray | None = None, select_bias: np.ndarray | None = None):
    """One MoE layer on FP32 activations x32 [T,H].  Routing runs for every token;
    the expert MLPs and the combine run for `token_subset` (all tokens if None).
    Returns dict(ids, w, y [n,H] float64, tokens)."""
    z = router_logits(x32, w_router, bias)
    ids, w = route(z, G, Kg, K, alpha, select_bias=select_bias)
    tok = np.arange(x32.shape[0]) if token_subset is None else np.asarray(token_subset)
    y = moe_combine(x32[tok].astype(np.float64), ids[tok], w[tok], bank)
    return {"ids": ids, "w": w, "y": y, "tokens": tok, "logits": z}


def sublayer_forward(h32: np.ndarray, pre_gain, post_gain, step_k: int, eps: float,
                     w_router, bias, bank: ExpertBank, G, Kg, K, alpha,
                     token_subset: np.ndarray | None = None, select_bias: np.ndarray | None = None):
    """pre-RMSNorm (FP32, fixed order) -> MoE -> post-RMSNorm -> constant-scale residual.
    Returns dict(ids, w, y (MoE output), h_new (float64), tokens)."""
    xhat, _ = prenorm(h32, pre_gain, eps)
    r = moe_forward(xhat, w_router, bias, bank, G, Kg, K, alpha, token_subset, select_bias)
    tok = r["tokens"]
    r["h_new"] = sublayer_output(h32[tok], r["y"], post_gain, step_k, eps)
    r["xhat"] = xhat
    return r


# ---------------------------------------------------------------------------
# dense SwiGLU MLP of the first decoder layers
# ---------------------------------------------------------------------------
def dense_forward(x32: np.ndarray, bank: ExpertBank, token_subset: np.ndarray | None = None):
    """Dense SwiGLU MLP (Reflection Beam 1.0 overview, "Architecture": the first 3 of the
    52 decoder layers run a dense SwiGLU MLP where the others run the MoE block):
    y[t] = Wd (SiLU(Wg x_t) * (Wu x_t)) in float64, with the single weight set held in
    slot 0 of `bank` (w13 [1, 2I, H], w2 [1, H, I], the layouts of one expert).  No
    router and no combine weight.  The dense width I is not on the pages.
    Returns dict(y [n,H] float64, tokens)."""
    tok = np.arange(x32.shape[0]) if token_subset is None else np.asarray(token_subset)
    w13, w2 = bank.expert(0)
    y = expert_ffn(x32[tok].astype(np.float64), w13, w2, bank.act_quant)
    return {"y": y, "tokens": tok}


def dense_sublayer_forward(h32: np.ndarray, pre_gain, post_gain, step_k: int, eps: float,
                           bank: ExpertBank, token_subset: np.ndarray | None = None):
    """pre-RMSNorm (FP32, fixed order) -> dense SwiGLU MLP -> post-RMSNorm ->
    constant-scale residual: the MoE sublayer with the dense MLP in the middle (the
    pages normalise every sublayer before and after).
    Returns dict(y (MLP output), h_new (float64), tokens, xhat)."""
    xhat, _ = prenorm(h32, pre_gain, eps)
    r = dense_forward(xhat, bank, token_subset)
    tok = r["tokens"]
    r["h_new"] = sublayer_output(h32[tok], r["y"], post_gain, step_k, eps)
    r["xhat"] = xhat
    return r
