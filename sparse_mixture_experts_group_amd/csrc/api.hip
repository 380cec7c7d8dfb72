// C ABI of libbeam_moe: validation, workspace layout and kernel sequencing.
// The declarations and the full contract of every entry point are in beam_moe.h.
#include <math.h>
#include <algorithm>
#include <mutex>
#include <set>
#include <string.h>
#include <utility>

#include "beam_moe.h"
#include "kernels.h"

using namespace beam;

namespace beam {

void lds_opt_in(const void* kernel, int bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    static std::mutex mu;
    static std::set<std::pair<const void*, int>> done;
    std::lock_guard<std::mutex> lock(mu);
    if (done.emplace(kernel, dev).second)
        (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

}  // namespace beam

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Structural validity of the configuration (independent of kernel support).
bool config_valid(const beam_moe_config* c) {
    if (!c) return false;
    if (c->hidden < 1 || c->inter < 1) return false;
    if (c->n_experts < 2 || c->n_experts > kMaxExperts) return false;
    if (c->n_groups < 1 || c->n_experts % c->n_groups != 0) return false;
    const int S = c->n_experts / c->n_groups;
    if (S < 2) return false;
    if (c->topk_groups < 1 || c->topk_groups > c->n_groups) return false;
    if (c->topk < 1 || c->topk > kMaxTopK || c->topk > c->topk_groups * S) return false;
    if (!isfinite(c->routed_scale)) return false;
    if (c->act_dtype < BEAM_DTYPE_F32 || c->act_dtype > BEAM_DTYPE_FP8_E4M3) return false;
    if (c->weight_dtype < BEAM_DTYPE_F32 || c->weight_dtype > BEAM_DTYPE_MXFP4) return false;
    if (!(c->norm_eps >= 0.0f) || !isfinite(c->norm_eps)) return false;
    if (c->fp8_scale_kind != BEAM_FP8_SCALES_FP32 && c->fp8_scale_kind != BEAM_FP8_SCALES_POW2) return false;
    return true;
}

// Whether the expert GEMM kernels cover these dtypes and shapes (shared by the MoE layer
// and the dense MLP).
bool gemm_supported(const beam_moe_config* c) {
    const int a = c->act_dtype, w = c->weight_dtype;
    const bool pair_ok = (a == BEAM_DTYPE_F32 && w == BEAM_DTYPE_F32) ||
                         (a == BEAM_DTYPE_BF16 && w == BEAM_DTYPE_BF16) ||
                         (a == BEAM_DTYPE_BF16 && w == BEAM_DTYPE_FP8_E4M3) ||
                         (a == BEAM_DTYPE_BF16 && w == BEAM_DTYPE_MXFP4);
    if (!pair_ok) return false;
    // LDS staging of the small-batch router and of the norms: at most 16384 columns
    if (c->hidden > 16384) return false;
    if (w == BEAM_DTYPE_F32) {
        if (c->hidden % 64 || c->inter % 64) return false;
    } else {
        // the prefill down GEMM covers the hidden dimension in 256-column tiles
        if (c->hidden % 256 || c->inter % 128) return false;
    }
    if (w == BEAM_DTYPE_FP8_E4M3 && c->fp8_block != 128) return false;
    return true;
}

// Whether kernels exist for this (valid) configuration.
bool config_supported(const beam_moe_config* c) {
    if (!gemm_supported(c)) return false;
    const int V = scores_per_lane(c->n_experts);
    const int S = c->n_experts / c->n_groups;
    if (S % V != 0 || !is_pow2(S / V)) return false;
    if (c->n_groups > 64) return false;
    return true;
}

struct Layout {
    size_t z, scores, zpart, ids, wts, blk_cnt, blk_off, pair_rank, exp_cnt, exp_off, tiles, meta, active;
    size_t row_of_pair, pair_of_row, xhat32, x16, x8, x8s, hbuf, h8, h8s, yperm, part;
    size_t total;
    int nblk, max_tiles, bm;
};

// Slices the dense MLP's MXFP4 down GEMM needs above the streaming range, where a
// slice's weight scales are staged in LDS (power of two).
int dense_mxfp4_min_slices(const beam_moe_config& c) {
    int s = 1;
    while (c.inter / s > kMxfp4PrefillMaxKd) s *= 2;
    return s;
}

// FP32 split-K partial sums of the dense MLP's GEMMs: half its gate/up weight bytes, or
// four [T, H] slices (the down GEMM of a long prefill), whichever is larger.  The
// launchers split while the grid holds fewer than four tiles per CU and the slices fit.
int64_t dense_part_floats(const beam_moe_config& c, int64_t T) {
    const double wb = c.weight_dtype == BEAM_DTYPE_BF16 ? 2.0 : (c.weight_dtype == BEAM_DTYPE_FP8_E4M3 ? 1.0 : 0.5);
    int64_t f = static_cast<int64_t>(2.0 * c.inter * c.hidden * wb / 2.0 / sizeof(float));
    f = std::max(f, 4 * T * c.hidden);
    if (c.weight_dtype == BEAM_DTYPE_MXFP4) f = std::max(f, dense_mxfp4_min_slices(c) * T * c.hidden);
    return (f + 63) / 64 * 64;
}

// Workspace regions.  dense: the dense MLP (c has n_experts = topk = 1): no router
// regions, and FP32 split-K partial sums for its GEMMs.
Layout make_layout(const beam_moe_config& c, int64_t T, bool dense = false) {
    Layout L;
    const int64_t E = c.n_experts, K = c.topk, H = c.hidden, I = c.inter;
    const int64_t P = T * K;
    const bool f32 = c.weight_dtype == BEAM_DTYPE_F32;
    // FP8 and MXFP4 weights take E4M3 activations (row-scaled copies of x and h)
    const bool fp8 = c.weight_dtype == BEAM_DTYPE_FP8_E4M3 || c.weight_dtype == BEAM_DTYPE_MXFP4;
    const bool bf16_act = c.act_dtype == BEAM_DTYPE_BF16;
    L.nblk = static_cast<int>((T + kSelectTokens - 1) / kSelectTokens);
    L.bm = kPrefillBM;
    L.max_tiles = static_cast<int>((P + L.bm - 1) / L.bm + E);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
    L.z = take(dense ? 0 : sizeof(float) * T * E);
    L.scores = take(dense ? 0 : sizeof(float) * T * E);
    // chunk sums of the small-T router kernel (only used below the tiled kernel's range)
    L.zpart = take((!dense && router_uses_partials(T, static_cast<int>(H), static_cast<int>(E)))
                       ? sizeof(float) * 64 * T * E : 0);
    L.ids = take(sizeof(int32_t) * P);
    L.wts = take(sizeof(float) * P);
    L.blk_cnt = take(dense ? 0 : sizeof(int32_t) * L.nblk * E);
    L.blk_off = take(dense ? 0 : sizeof(int32_t) * L.nblk * E);
    L.pair_rank = take(dense ? 0 : sizeof(int32_t) * P);
    L.exp_cnt = take(sizeof(int32_t) * E);
    L.exp_off = take(sizeof(int32_t) * (E + 1));
    L.tiles = take(sizeof(int2) * L.max_tiles);
    L.meta = take(sizeof(int32_t) * kMetaInts);
    L.active = take(sizeof(int32_t) * E);
    L.row_of_pair = take(sizeof(int32_t) * P);
    L.pair_of_row = take(sizeof(int32_t) * P);
    // sublayer (BF16 residual stream): FP32 normalised input for the router, and the
    // expert input in the weights' format
    L.xhat32 = (bf16_act && !dense) ? take(sizeof(float) * T * H) : off;
    L.x16 = (bf16_act && !fp8) ? take(sizeof(uint16_t) * T * H) : off;
    L.x8 = fp8 ? take(T * H) : off;
    L.x8s = fp8 ? take(sizeof(float) * T) : off;
    L.hbuf = take((f32 ? 4 : 2) * P * I);
    L.h8 = fp8 ? take(P * I) : off;
    L.h8s = fp8 ? take(sizeof(float) * P) : off;
    L.yperm = take((f32 ? 4 : 2) * P * H);
    // split-K partial sums of the dense MLP
    L.part = take((dense && !f32) ? dense_part_floats(c, T) * sizeof(float) : 0);
    L.total = off;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int check_common(const beam_moe_config* cfg, int64_t T) {
    if (!config_valid(cfg) || T < 0) return BEAM_ERR_INVALID_ARG;
    if (T > 0 && T * cfg->topk > INT32_MAX / 2) return BEAM_ERR_INVALID_ARG;
    if (!config_supported(cfg)) return BEAM_ERR_UNSUPPORTED;
    return BEAM_OK;
}

int check_ws(const beam_moe_config* cfg, int64_t T, void* ws, size_t ws_bytes) {
    const Layout L = make_layout(*cfg, T);
    if (!ws || ws_bytes < L.total) return BEAM_ERR_WORKSPACE;
    if (!aligned16(ws)) return BEAM_ERR_INVALID_ARG;
    return BEAM_OK;
}

// Kernel timing hook state (see beam_moe_time_kernel): one per host thread, so threads
// that drive different devices (or streams) time their own launches without racing.
struct TimingHook {
    int kernel = BEAM_KERNEL_NONE;
    void* const* events = nullptr;
    int n_pairs = 0;
    int next = 0;
};
thread_local TimingHook g_hook;

struct Bracket {
    hipStream_t st;
    hipEvent_t stop = nullptr;
    Bracket(int kernel, hipStream_t s) : st(s) {
        if (g_hook.kernel == kernel && g_hook.next < g_hook.n_pairs) {
            const int i = g_hook.next++;
            (void)hipEventRecord(static_cast<hipEvent_t>(g_hook.events[2 * i]), st);
            stop = static_cast<hipEvent_t>(g_hook.events[2 * i + 1]);
        }
    }
    ~Bracket() {
        if (stop) (void)hipEventRecord(stop, st);
    }
};

// Clears the thread's last-HIP-error state right before the first enqueue, so that the
// status check after the launches reports only this call's launch failures.
void clear_hip_error() { (void)hipGetLastError(); }

int launch_status() {
    return hipGetLastError() == hipSuccess ? BEAM_OK : BEAM_ERR_HIP;
}

// Router + permutation.  x_router is FP32 or BF16 [T, H].
void run_router(const beam_moe_config& c, int64_t T, const Layout& L, void* ws, hipStream_t st,
                const void* x_router, bool x_bf16, const float* w_router, const float* bias,
                const float* select_bias, int32_t* ids, float* wts, bool permute) {
    const int E = c.n_experts, K = c.topk;
    float* z = at<float>(ws, L.z);
    {
        Bracket b(BEAM_KERNEL_ROUTER_LOGITS, st);
        launch_router_logits(st, static_cast<int>(T), c.hidden, E, x_bf16, x_router, w_router, bias, z,
                             at<float>(ws, L.zpart));
    }
    launch_router_select(st, static_cast<int>(T), E, c.n_groups, c.topk_groups, K, c.routed_scale, z, select_bias,
                         ids, wts, at<int32_t>(ws, L.blk_cnt), at<int32_t>(ws, L.pair_rank), at<float>(ws, L.scores));
    if (!permute) return;
    if (L.nblk <= kFinishSmallBlocks) {
        launch_route_finish_small(st, static_cast<int>(T), K, E, L.nblk, L.bm, ids, at<int32_t>(ws, L.pair_rank),
                                  at<int32_t>(ws, L.blk_cnt), at<int32_t>(ws, L.blk_off), at<int32_t>(ws, L.exp_cnt),
                                  at<int32_t>(ws, L.exp_off), at<int2>(ws, L.tiles), at<int32_t>(ws, L.meta),
                                  at<int32_t>(ws, L.active), at<int32_t>(ws, L.row_of_pair),
                                  at<int32_t>(ws, L.pair_of_row));
        return;
    }
    launch_route_scan(st, L.nblk, E, L.bm, at<int32_t>(ws, L.blk_cnt), at<int32_t>(ws, L.blk_off),
                      at<int32_t>(ws, L.exp_cnt), at<int32_t>(ws, L.exp_off), at<int2>(ws, L.tiles),
                      at<int32_t>(ws, L.meta), at<int32_t>(ws, L.active));
    launch_route_scatter(st, T * K, K, E, ids, at<int32_t>(ws, L.pair_rank), at<int32_t>(ws, L.blk_off),
                         at<int32_t>(ws, L.exp_off), at<int32_t>(ws, L.row_of_pair), at<int32_t>(ws, L.pair_of_row));
}

GroupedGemmArgs base_args(const beam_moe_config& c, int64_t T, const Layout& L, void* ws) {
    GroupedGemmArgs g;
    memset(&g, 0, sizeof(g));
    g.pair_of_row = at<int32_t>(ws, L.pair_of_row);
    g.topk = c.topk;
    g.exp_cnt = at<int32_t>(ws, L.exp_cnt);
    g.exp_off = at<int32_t>(ws, L.exp_off);
    g.tiles = at<int2>(ws, L.tiles);
    g.meta = at<int32_t>(ws, L.meta);
    g.active = at<int32_t>(ws, L.active);
    g.max_tiles = L.max_tiles;
    const int64_t P = T * c.topk;
    // Few rows per expert (weight streaming): pairs of row tiles share an XCD's L2 slice
    // with more column tiles; many rows (MFMA-bound): groups of 4 share weight panels.
    g.group_m = (P >= 512LL * c.n_experts) ? 4 : 2;
    g.max_active = static_cast<int>(P < c.n_experts ? P : c.n_experts);
    g.max_rows = static_cast<int>(T);     // a token picks an expert at most once
    g.w_scale_pow2 = c.weight_dtype == BEAM_DTYPE_FP8_E4M3 && c.fp8_scale_kind == BEAM_FP8_SCALES_POW2;
    return g;
}

// LDS-tiled GEMMs: the 128-byte-stage kernel (gemm_wide.hip) for BF16 and FP8 weights,
// the 128-value-stage kernel (gemm_wide_mx.hip) for MXFP4 weights while a K slice fits
// its LDS scale budget; both address their operands with 32-bit offsets and take FP8
// reductions of at most 64 scale blocks.  The 64-byte-stage kernel (gemm_prefill.hip)
// serves the rest.  a_rows: rows of the activation matrix.
int launch_tiled(hipStream_t st, GemmMode mode, const GroupedGemmArgs& ga, PrefillWeights wt, int64_t a_rows) {
    GroupedGemmArgs g = ga;
    g.a_rows = a_rows;
    const int64_t nw = (mode == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const bool fits = a_rows * g.lda * 2 < (int64_t{1} << 32) && nw * g.kd * 2 < (int64_t{1} << 32);
    if (wt == PrefillWeights::kBf16 && fits) return launch_gemm_wide(st, mode, g, false);
    if (wt == PrefillWeights::kFp8 && g.kd <= 64 * 128 && fits) return launch_gemm_wide(st, mode, g, true);
    if (wt == PrefillWeights::kMxfp4 && fits) {
        const int ks = prefill_k_split(mode, g, wt);
        if (wide_mx_supported(g, ks)) return launch_gemm_wide_mx(st, mode, g, ks);
    }
    return launch_gemm_prefill(st, mode, g, wt);
}

// Expert GEMMs: x_exp [T, H] in the weights' activation format -> down_out [T*K, H]
// (yperm for the MoE layer).  dense: the single weight set of the dense MLP (rows are
// tokens, no gather), whose streaming down GEMM may split K into FP32 partial sums that
// one more kernel adds up.
// Largest token count at which GEMM `mode` runs on the streaming kernels.
int64_t stream_max_t(const beam_moe_config& c, bool dense, GemmMode mode) {
    if (dense) return kDenseStreamMaxT;
    if (c.weight_dtype == BEAM_DTYPE_MXFP4) return kDecodeMaxT;
    if (c.weight_dtype == BEAM_DTYPE_FP8_E4M3) return mode == kGateUp ? kFp8GateUpStreamMaxT : kFp8DownStreamMaxT;
    return mode == kGateUp ? kBf16GateUpStreamMaxT : kBf16DownStreamMaxT;
}

void run_experts(const beam_moe_config& c, int64_t T, const Layout& L, void* ws, hipStream_t st,
                 const void* x_exp, const float* x_exp_scale, const void* w13,
                 const void* w13_scale, const void* w2, const void* w2_scale,
                 const int32_t* ids, void* down_out, bool dense = false) {
    const int64_t P = T * c.topk;
    const int H = c.hidden, I = c.inter;
    GroupedGemmArgs g1 = base_args(c, T, L, ws);
    g1.a = x_exp; g1.lda = H; g1.gather = !dense; g1.a_scale = x_exp_scale;
    g1.w = w13; g1.w_scale = w13_scale; g1.n_out = I; g1.kd = H;
    g1.out = at<void>(ws, L.hbuf); g1.ldo = I;
    GroupedGemmArgs g2 = base_args(c, T, L, ws);
    g2.lda = I; g2.gather = false;
    g2.w = w2; g2.w_scale = w2_scale; g2.n_out = H; g2.kd = I;
    g2.out = down_out; g2.ldo = H;
    // streaming kernels while the rows of an expert are few (measured crossovers, per
    // GEMM): T tokens spread over the experts, or at most 16 rows of the dense MLP's
    // single weight set (the streaming kernels read the weights once per 32 rows)
    const bool decode1 = T <= stream_max_t(c, dense, kGateUp);
    const bool decode2 = T <= stream_max_t(c, dense, kDown);
    if (dense && c.weight_dtype != BEAM_DTYPE_F32) {
        g1.part = g2.part = at<float>(ws, L.part);
        g1.part_cap = g2.part_cap = dense_part_floats(c, T);
        g1.part_slice = P * 2 * I;
        g2.part_slice = P * H;
    }
    int slices = 1, slices1 = 1;
    // after a split gate/up GEMM: the SwiGLU of the summed partials into hbuf
    auto swiglu = [&]() {
        if (slices1 > 1)
            launch_splitk_swiglu(st, slices1, P, I, g1.part_slice, g1.part, at<uint16_t>(ws, L.hbuf));
    };
    if (c.weight_dtype == BEAM_DTYPE_F32) {
        { Bracket b(BEAM_KERNEL_GATE_UP, st); launch_gemm_f32(st, kGateUp, g1, P, ids); }
        g2.a = at<void>(ws, L.hbuf);
        { Bracket b(BEAM_KERNEL_DOWN, st); launch_gemm_f32(st, kDown, g2, P, ids); }
    } else if (c.weight_dtype == BEAM_DTYPE_BF16) {
        {
            Bracket b(BEAM_KERNEL_GATE_UP, st);
            if (decode1) slices1 = launch_gemm_bf16_decode(st, kGateUp, g1);
            else slices1 = launch_tiled(st, kGateUp, g1, PrefillWeights::kBf16, T);
        }
        swiglu();
        g2.a = at<void>(ws, L.hbuf);
        {
            Bracket b(BEAM_KERNEL_DOWN, st);
            if (decode2) slices = launch_gemm_bf16_decode(st, kDown, g2);
            else slices = launch_tiled(st, kDown, g2, PrefillWeights::kBf16, P);
        }
    } else if (c.weight_dtype == BEAM_DTYPE_FP8_E4M3) {
        {
            Bracket b(BEAM_KERNEL_GATE_UP, st);
            if (decode1) slices1 = launch_gemm_fp8_decode(st, kGateUp, g1);
            else slices1 = launch_tiled(st, kGateUp, g1, PrefillWeights::kFp8, T);
        }
        swiglu();
        launch_quant_rows_fp8(st, P, I, true, at<void>(ws, L.hbuf), at<uint8_t>(ws, L.h8), at<float>(ws, L.h8s));
        g2.a = at<void>(ws, L.h8); g2.a_scale = at<float>(ws, L.h8s);
        {
            Bracket b(BEAM_KERNEL_DOWN, st);
            if (decode2) slices = launch_gemm_fp8_decode(st, kDown, g2);
            else slices = launch_tiled(st, kDown, g2, PrefillWeights::kFp8, P);
        }
    } else {            // MXFP4 weights
        {
            Bracket b(BEAM_KERNEL_GATE_UP, st);
            if (decode1) slices1 = launch_gemm_mxfp4_decode(st, kGateUp, g1);
            else slices1 = launch_tiled(st, kGateUp, g1, PrefillWeights::kMxfp4, T);
        }
        swiglu();
        launch_quant_rows_fp8(st, P, I, true, at<void>(ws, L.hbuf), at<uint8_t>(ws, L.h8), at<float>(ws, L.h8s));
        g2.a = at<void>(ws, L.h8); g2.a_scale = at<float>(ws, L.h8s);
        {
            Bracket b(BEAM_KERNEL_DOWN, st);
            if (decode2) slices = launch_gemm_mxfp4_decode(st, kDown, g2);
            else slices = launch_tiled(st, kDown, g2, PrefillWeights::kMxfp4, P);
        }
    }
    if (slices > 1) launch_splitk_reduce(st, slices, P * H, g2.part_slice, g2.part, static_cast<uint16_t*>(down_out));
}

}  // namespace

extern "C" {

const char* beam_moe_status_string(int status) {
    switch (status) {
        case BEAM_OK: return "BEAM_OK";
        case BEAM_ERR_INVALID_ARG: return "BEAM_ERR_INVALID_ARG: null pointer, bad shape or bad config";
        case BEAM_ERR_UNSUPPORTED: return "BEAM_ERR_UNSUPPORTED: no kernels for this configuration";
        case BEAM_ERR_WORKSPACE: return "BEAM_ERR_WORKSPACE: workspace missing or smaller than beam_moe_workspace_size()";
        case BEAM_ERR_HIP: return "BEAM_ERR_HIP: a kernel launch failed";
        default: return "unknown beam_status";
    }
}

int beam_moe_abi_version(void) { return BEAM_MOE_ABI_VERSION; }

size_t beam_moe_workspace_size(const beam_moe_config* cfg, int64_t T) {
    if (!config_valid(cfg) || T < 0) return 0;
    return make_layout(*cfg, T).total;
}

int beam_moe_workspace_map(const beam_moe_config* cfg, int64_t T, beam_moe_ws_map* out) {
    if (!config_valid(cfg) || T < 0 || !out) return BEAM_ERR_INVALID_ARG;
    const Layout L = make_layout(*cfg, T);
    out->logits = L.z;
    out->expert_count = L.exp_cnt;
    out->expert_off = L.exp_off;
    out->row_of_pair = L.row_of_pair;
    out->pair_of_row = L.pair_of_row;
    out->hidden = L.hbuf;
    out->expert_out = L.yperm;
    out->scores = L.scores;
    out->xhat = L.xhat32;
    out->x_q = L.x8;
    out->x_q_scale = L.x8s;
    out->h_q = L.h8;
    out->h_q_scale = L.h8s;
    out->total = L.total;
    return BEAM_OK;
}

int beam_moe_route(const beam_moe_config* cfg, int64_t T, const void* x, const float* w_router,
                   const float* logit_bias, const float* select_bias, int32_t* ids, float* weights, void* ws,
                   size_t ws_bytes, void* stream) {
    int s = check_common(cfg, T);
    if (s != BEAM_OK) return s;
    if (cfg->act_dtype == BEAM_DTYPE_FP8_E4M3) return BEAM_ERR_UNSUPPORTED;
    if (T == 0) return BEAM_OK;
    if (!x || !w_router || !ids || !weights) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router)) return BEAM_ERR_INVALID_ARG;
    if ((s = check_ws(cfg, T, ws, ws_bytes)) != BEAM_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = make_layout(*cfg, T);
    clear_hip_error();
    run_router(*cfg, T, L, ws, st, x, cfg->act_dtype == BEAM_DTYPE_BF16, w_router, logit_bias, select_bias, ids,
               weights, false);
    return launch_status();
}

static int check_weights(const beam_moe_config* cfg, int64_t T, const void* w13, const void* w13_scale,
                         const void* w2, const void* w2_scale, bool dense = false) {
    if (!w13 || !w2) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(w13) || !aligned16(w2)) return BEAM_ERR_INVALID_ARG;
    const bool scaled = cfg->weight_dtype == BEAM_DTYPE_FP8_E4M3 || cfg->weight_dtype == BEAM_DTYPE_MXFP4;
    if (scaled != (w13_scale != nullptr) || scaled != (w2_scale != nullptr)) return BEAM_ERR_INVALID_ARG;
    if (scaled && (!aligned16(w13_scale) || !aligned16(w2_scale))) return BEAM_ERR_INVALID_ARG;
    // GEMMs above their streaming range run LDS-tiled (gate/up reduces over hidden, down
    // over inter)
    const bool tiled1 = T > stream_max_t(*cfg, dense, kGateUp);
    const bool tiled2 = T > stream_max_t(*cfg, dense, kDown);
    if (cfg->weight_dtype == BEAM_DTYPE_MXFP4) {
        // MXFP4 tiles stage their weight scales in LDS; the dense MLP's down GEMM splits K
        // into slices whose scales fit
        if (tiled1 && cfg->hidden > kMxfp4PrefillMaxKd) return BEAM_ERR_UNSUPPORTED;
        if (tiled2 && dense) {
            const int ms = dense_mxfp4_min_slices(*cfg);
            if (ms > kMaxKSplit || cfg->inter % (ms * 512) != 0) return BEAM_ERR_UNSUPPORTED;
        } else if (tiled2 && cfg->inter > kMxfp4PrefillMaxKd) {
            return BEAM_ERR_UNSUPPORTED;
        }
    }
    // FP8 tiles hold the K-block scale codes of one reduction in LDS
    if (cfg->weight_dtype == BEAM_DTYPE_FP8_E4M3 &&
        ((tiled1 && cfg->hidden > kFp8PrefillMaxKd) || (tiled2 && cfg->inter > kFp8PrefillMaxKd)))
        return BEAM_ERR_UNSUPPORTED;
    return BEAM_OK;
}

int beam_moe_forward(const beam_moe_config* cfg, int64_t T, const void* x, const float* w_router,
                     const float* logit_bias, const float* select_bias, const void* w13,
                     const void* w13_scale, const void* w2,
                     const void* w2_scale, void* y, int32_t* ids_out, float* weights_out, void* ws,
                     size_t ws_bytes, void* stream) {
    int s = check_common(cfg, T);
    if (s != BEAM_OK) return s;
    if (T == 0) return BEAM_OK;
    if (!x || !w_router || !y) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(y)) return BEAM_ERR_INVALID_ARG;
    if ((s = check_weights(cfg, T, w13, w13_scale, w2, w2_scale)) != BEAM_OK) return s;
    if ((s = check_ws(cfg, T, ws, ws_bytes)) != BEAM_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = make_layout(*cfg, T);
    clear_hip_error();
    int32_t* ids = ids_out ? ids_out : at<int32_t>(ws, L.ids);
    float* wts = weights_out ? weights_out : at<float>(ws, L.wts);
    const bool bf16_act = cfg->act_dtype == BEAM_DTYPE_BF16;
    run_router(*cfg, T, L, ws, st, x, bf16_act, w_router, logit_bias, select_bias, ids, wts, true);
    const void* x_exp = x;
    const float* x_exp_scale = nullptr;
    if (cfg->weight_dtype == BEAM_DTYPE_FP8_E4M3 || cfg->weight_dtype == BEAM_DTYPE_MXFP4) {
        launch_quant_rows_fp8(st, T, cfg->hidden, true, x, at<uint8_t>(ws, L.x8), at<float>(ws, L.x8s));
        x_exp = at<void>(ws, L.x8);
        x_exp_scale = at<float>(ws, L.x8s);
    }
    run_experts(*cfg, T, L, ws, st, x_exp, x_exp_scale, w13, w13_scale, w2, w2_scale, ids, at<void>(ws, L.yperm));
    Bracket b(BEAM_KERNEL_COMBINE, st);
    launch_combine(st, T, cfg->hidden, cfg->topk, cfg->weight_dtype == BEAM_DTYPE_F32, at<void>(ws, L.yperm),
                   at<int32_t>(ws, L.row_of_pair), wts, y);
    return launch_status();
}

int beam_moe_sublayer_forward(const beam_moe_config* cfg, int64_t T, void* h, const float* pre_gain,
                              const float* post_gain, int32_t step_k, const float* w_router,
                              const float* logit_bias, const float* select_bias, const void* w13,
                              const void* w13_scale,
                              const void* w2, const void* w2_scale, void* moe_out, int32_t* ids_out,
                              float* weights_out, void* ws, size_t ws_bytes, void* stream) {
    int s = check_common(cfg, T);
    if (s != BEAM_OK) return s;
    if (cfg->act_dtype != BEAM_DTYPE_BF16) return BEAM_ERR_UNSUPPORTED;
    if (step_k < 2) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!h || !w_router) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(h) || !aligned16(w_router) || (moe_out && !aligned16(moe_out))) return BEAM_ERR_INVALID_ARG;
    if ((s = check_weights(cfg, T, w13, w13_scale, w2, w2_scale)) != BEAM_OK) return s;
    if ((s = check_ws(cfg, T, ws, ws_bytes)) != BEAM_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = make_layout(*cfg, T);
    clear_hip_error();
    int32_t* ids = ids_out ? ids_out : at<int32_t>(ws, L.ids);
    float* wts = weights_out ? weights_out : at<float>(ws, L.wts);
    // E4M3 activations for FP8 and MXFP4 weights
    const bool fp8 = cfg->weight_dtype == BEAM_DTYPE_FP8_E4M3 || cfg->weight_dtype == BEAM_DTYPE_MXFP4;
    const int H = cfg->hidden;
    launch_prenorm(st, T, H, static_cast<const uint16_t*>(h), pre_gain, cfg->norm_eps, at<float>(ws, L.xhat32),
                   fp8 ? nullptr : at<uint16_t>(ws, L.x16), fp8 ? at<uint8_t>(ws, L.x8) : nullptr,
                   fp8 ? at<float>(ws, L.x8s) : nullptr);
    run_router(*cfg, T, L, ws, st, at<float>(ws, L.xhat32), false, w_router, logit_bias, select_bias, ids, wts,
               true);
    const void* x_exp = fp8 ? at<void>(ws, L.x8) : at<void>(ws, L.x16);
    const float* x_exp_scale = fp8 ? at<float>(ws, L.x8s) : nullptr;
    run_experts(*cfg, T, L, ws, st, x_exp, x_exp_scale, w13, w13_scale, w2, w2_scale, ids, at<void>(ws, L.yperm));
    // c1 = sqrt((k-1)/k), c2 = 1/sqrt(k), each computed in double and rounded once
    const double k = static_cast<double>(step_k);
    const float c1 = static_cast<float>(sqrt((k - 1.0) / k));
    const float c2 = static_cast<float>(1.0 / sqrt(k));
    Bracket b(BEAM_KERNEL_COMBINE, st);
    launch_post_residual(st, T, H, cfg->topk, at<uint16_t>(ws, L.yperm), at<int32_t>(ws, L.row_of_pair), wts,
                         post_gain, cfg->norm_eps, c1, c2, static_cast<uint16_t*>(h),
                         static_cast<uint16_t*>(moe_out));
    return launch_status();
}

// The dense MLP runs on the MoE machinery as one expert that every token picks once
// with weight 1; of cfg only hidden, inter, act_dtype, weight_dtype, fp8_block and
// norm_eps are read.
static beam_moe_config dense_view(const beam_moe_config* cfg) {
    beam_moe_config c = *cfg;
    c.n_experts = 1;
    c.n_groups = 1;
    c.topk_groups = 1;
    c.topk = 1;
    c.routed_scale = 1.0f;
    return c;
}

static bool dense_config_valid(const beam_moe_config* c) {
    if (!c) return false;
    if (c->hidden < 1 || c->inter < 1) return false;
    if (c->act_dtype < BEAM_DTYPE_F32 || c->act_dtype > BEAM_DTYPE_FP8_E4M3) return false;
    if (c->weight_dtype < BEAM_DTYPE_F32 || c->weight_dtype > BEAM_DTYPE_MXFP4) return false;
    if (!(c->norm_eps >= 0.0f) || !isfinite(c->norm_eps)) return false;
    if (c->fp8_scale_kind != BEAM_FP8_SCALES_FP32 && c->fp8_scale_kind != BEAM_FP8_SCALES_POW2) return false;
    return true;
}

static int check_dense(const beam_moe_config* cfg, int64_t T) {
    if (!dense_config_valid(cfg) || T < 0 || T > INT32_MAX / 2) return BEAM_ERR_INVALID_ARG;
    const beam_moe_config c = dense_view(cfg);
    if (!gemm_supported(&c)) return BEAM_ERR_UNSUPPORTED;
    return BEAM_OK;
}

static int check_dense_ws(const beam_moe_config& c, int64_t T, void* ws, size_t ws_bytes) {
    if (!ws || ws_bytes < make_layout(c, T, true).total) return BEAM_ERR_WORKSPACE;
    if (!aligned16(ws)) return BEAM_ERR_INVALID_ARG;
    return BEAM_OK;
}

static void dense_tables(int64_t T, const Layout& L, void* ws, hipStream_t st) {
    launch_dense_setup(st, T, L.bm, at<int32_t>(ws, L.ids), at<int32_t>(ws, L.exp_cnt), at<int32_t>(ws, L.exp_off),
                       at<int2>(ws, L.tiles), at<int32_t>(ws, L.meta), at<int32_t>(ws, L.active),
                       at<int32_t>(ws, L.row_of_pair), at<int32_t>(ws, L.pair_of_row), at<float>(ws, L.wts));
}

size_t beam_dense_workspace_size(const beam_moe_config* cfg, int64_t T) {
    if (!dense_config_valid(cfg) || T < 0 || T > INT32_MAX / 2) return 0;
    return make_layout(dense_view(cfg), T, true).total;
}

int beam_dense_forward(const beam_moe_config* cfg, int64_t T, const void* x, const void* w13,
                       const void* w13_scale, const void* w2, const void* w2_scale, void* y, void* ws,
                       size_t ws_bytes, void* stream) {
    int s = check_dense(cfg, T);
    if (s != BEAM_OK) return s;
    if (T == 0) return BEAM_OK;
    if (!x || !y) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y)) return BEAM_ERR_INVALID_ARG;
    const beam_moe_config c = dense_view(cfg);
    if ((s = check_weights(&c, T, w13, w13_scale, w2, w2_scale, true)) != BEAM_OK) return s;
    if ((s = check_dense_ws(c, T, ws, ws_bytes)) != BEAM_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = make_layout(c, T, true);
    clear_hip_error();
    dense_tables(T, L, ws, st);
    const void* x_exp = x;
    const float* x_exp_scale = nullptr;
    if (c.weight_dtype == BEAM_DTYPE_FP8_E4M3 || c.weight_dtype == BEAM_DTYPE_MXFP4) {
        launch_quant_rows_fp8(st, T, c.hidden, true, x, at<uint8_t>(ws, L.x8), at<float>(ws, L.x8s));
        x_exp = at<void>(ws, L.x8);
        x_exp_scale = at<float>(ws, L.x8s);
    }
    run_experts(c, T, L, ws, st, x_exp, x_exp_scale, w13, w13_scale, w2, w2_scale, at<int32_t>(ws, L.ids), y, true);
    return launch_status();
}

int beam_dense_sublayer_forward(const beam_moe_config* cfg, int64_t T, void* h, const float* pre_gain,
                                const float* post_gain, int32_t step_k, const void* w13, const void* w13_scale,
                                const void* w2, const void* w2_scale, void* mlp_out, void* ws, size_t ws_bytes,
                                void* stream) {
    int s = check_dense(cfg, T);
    if (s != BEAM_OK) return s;
    if (cfg->act_dtype != BEAM_DTYPE_BF16) return BEAM_ERR_UNSUPPORTED;
    if (step_k < 2) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!h) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(h) || (mlp_out && !aligned16(mlp_out))) return BEAM_ERR_INVALID_ARG;
    const beam_moe_config c = dense_view(cfg);
    if ((s = check_weights(&c, T, w13, w13_scale, w2, w2_scale, true)) != BEAM_OK) return s;
    if ((s = check_dense_ws(c, T, ws, ws_bytes)) != BEAM_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = make_layout(c, T, true);
    clear_hip_error();
    dense_tables(T, L, ws, st);
    const bool fp8 = c.weight_dtype == BEAM_DTYPE_FP8_E4M3 || c.weight_dtype == BEAM_DTYPE_MXFP4;
    const int H = c.hidden;
    launch_prenorm(st, T, H, static_cast<const uint16_t*>(h), pre_gain, c.norm_eps, nullptr,
                   fp8 ? nullptr : at<uint16_t>(ws, L.x16), fp8 ? at<uint8_t>(ws, L.x8) : nullptr,
                   fp8 ? at<float>(ws, L.x8s) : nullptr);
    const void* x_exp = fp8 ? at<void>(ws, L.x8) : at<void>(ws, L.x16);
    const float* x_exp_scale = fp8 ? at<float>(ws, L.x8s) : nullptr;
    run_experts(c, T, L, ws, st, x_exp, x_exp_scale, w13, w13_scale, w2, w2_scale, at<int32_t>(ws, L.ids),
                at<void>(ws, L.yperm), true);
    const double k = static_cast<double>(step_k);
    const float c1 = static_cast<float>(sqrt((k - 1.0) / k));
    const float c2 = static_cast<float>(1.0 / sqrt(k));
    Bracket b(BEAM_KERNEL_COMBINE, st);
    launch_post_residual(st, T, H, 1, at<uint16_t>(ws, L.yperm), at<int32_t>(ws, L.row_of_pair),
                         at<float>(ws, L.wts), post_gain, c.norm_eps, c1, c2, static_cast<uint16_t*>(h),
                         static_cast<uint16_t*>(mlp_out));
    return launch_status();
}

}  // extern "C"

// The no-allocation forward's intermediates: one copy of this array per device.  In host
// code the name stands for a host-side shadow, not a device address: kernels are given
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[BEAM_MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BEAM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return BEAM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return BEAM_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BEAM_OK;
}

}  // namespace

extern "C" {

int beam_moe_forward_noalloc(const beam_moe_config* cfg, int64_t T, const void* x, const float* w_router,
                             const float* logit_bias, const float* select_bias, const void* w13,
                             const void* w13_scale, const void* w2, const void* w2_scale, void* y,
                             int32_t* ids_out, float* weights_out, void* stream) {
    int s = check_common(cfg, T);
    if (s != BEAM_OK) return s;
    if (T == 0) return BEAM_OK;
    if (make_layout(*cfg, T).total > BEAM_MOE_NOALLOC_SCRATCH_BYTES) return BEAM_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((s = scratch_address(&ws)) != BEAM_OK) return s;
    return beam_moe_forward(cfg, T, x, w_router, logit_bias, select_bias, w13, w13_scale, w2, w2_scale, y, ids_out,
                            weights_out, ws, BEAM_MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int beam_moe_time_kernel(int kernel, void* const* events, int n_pairs) {
    if (kernel < BEAM_KERNEL_NONE || kernel > BEAM_KERNEL_COMBINE || n_pairs < 0) return BEAM_ERR_INVALID_ARG;
    if (n_pairs > 0 && !events) return BEAM_ERR_INVALID_ARG;
    g_hook.kernel = (n_pairs > 0) ? kernel : BEAM_KERNEL_NONE;
    g_hook.events = events;
    g_hook.n_pairs = n_pairs;
    g_hook.next = 0;
    return BEAM_OK;
}

}  // extern "C"
