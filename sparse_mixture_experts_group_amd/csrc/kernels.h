// Internal launcher interface of libbeam_moe (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

constexpr int kSelectTokens = 16;   // tokens (one per wavefront) per selection block
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 256;
constexpr int kMetaTiles = 0;       // meta[0]: number of (expert, row-tile) tiles
constexpr int kMetaActive = 1;      // meta[1]: number of experts with >= 1 row
constexpr int kMetaInts = 64;

constexpr int kPrefillBM = 256;     // rows per tile of the prefill grouped GEMMs
// Tiles of an expert with n routed rows for the prefill GEMMs: ceil(n / BM) tiles of
// whole 32-row blocks, as equal as possible (so the tiles of one expert carry the same
// work and stream its weights in step).  Tile j holds rows [first(j), first(j + 1)),
// first(count) = n.  The tile list stores (expert, j).
__host__ __device__ inline int expert_tile_count(int n, int BM) { return (n + BM - 1) / BM; }
__host__ __device__ inline int expert_tile_first(int n, int j, int BM) {
    const int nt = expert_tile_count(n, BM);
    if (j >= nt) return n;
    const int64_t m = (n + 31) / 32;
    return static_cast<int>((j * m / nt) * 32);
}
// Token counts up to which a GEMM uses the streaming kernels (measured crossovers; the
// LDS-tiled kernels above): MXFP4 weights, both GEMMs
constexpr int kDecodeMaxT = 256;
// BF16 and FP8 weights, per GEMM (the tiled down GEMM, with I = 2560 columns of
// reduction, takes over later than the tiled gate/up GEMM)
constexpr int kBf16GateUpStreamMaxT = 32, kBf16DownStreamMaxT = 55;
constexpr int kFp8GateUpStreamMaxT = 16, kFp8DownStreamMaxT = 103;
constexpr int kDenseStreamMaxT = 16;   // the dense MLP (all rows on one weight set), both GEMMs

// The router logits use the chunk-parallel kernel (with a [64, T, E] FP32 scratch of
// chunk sums) below 1536 tokens and the matrix-core kernel from there on; the latter
// stages whole multiples of 16 hidden entries of one chunk (H / 64 % 16 == 0) and whole
// 128-expert blocks.  Measured crossover on the Beam router (one MI355X): 1024 tokens
// 0.11 against 0.13-0.14 ms, 1536 tokens 0.16 against 0.13-0.14, 4095 tokens 0.48
// against 0.23-0.26 (the matrix-core kernel's time is nearly flat below 2048 tokens,
// where it holds fewer waves than SIMDs).
inline bool router_uses_partials(int64_t T, int H, int E) {
    return !(E % 128 == 0 && T >= 1536 && (H / 64) % 16 == 0);
}

inline int scores_per_lane(int E) { return E <= 64 ? 1 : (E <= 128 ? 2 : 4); }

// Raises `kernel`'s dynamic-LDS limit to `bytes` on the current device, once per
// (kernel, device) in the process (the attribute belongs to a device).
void lds_opt_in(const void* kernel, int bytes);

enum GemmMode { kGateUp = 0, kDown = 1 };

// router.hip
// part: [64, T, E] FP32 scratch for the chunk sums of the small-T kernel
void launch_router_logits(hipStream_t st, int T, int H, int E, bool x_bf16, const void* x,
                          const float* wr, const float* bias, float* z, float* part);
// scores: [T, E] FP32 out, the sigmoid scores (for inspection)
void launch_router_select(hipStream_t st, int T, int E, int G, int Kg, int K, float alpha,
                          const float* z, const float* sel_bias, int32_t* ids, float* wts, int32_t* blk_cnt,
                          int32_t* pair_rank, float* scores);
void launch_route_scan(hipStream_t st, int nblk, int E, int BM, const int32_t* blk_cnt,
                       int32_t* blk_off, int32_t* exp_cnt, int32_t* exp_off, int2* tiles,
                       int32_t* meta, int32_t* active);
constexpr int kFinishSmallBlocks = 16;   // selection blocks handled by the fused finish kernel
void launch_route_finish_small(hipStream_t st, int T, int K, int E, int nblk, int BM, const int32_t* ids,
                               const int32_t* pair_rank, const int32_t* blk_cnt, int32_t* blk_off,
                               int32_t* exp_cnt, int32_t* exp_off, int2* tiles, int32_t* meta, int32_t* active,
                               int32_t* row_of_pair, int32_t* pair_of_row);
void launch_route_scatter(hipStream_t st, int64_t npairs, int K, int E, const int32_t* ids,
                          const int32_t* pair_rank, const int32_t* blk_off, const int32_t* exp_off,
                          int32_t* row_of_pair, int32_t* pair_of_row);

// Arguments shared by the grouped GEMM launchers.
struct GroupedGemmArgs {
    const void* a;            // activations: x [T, Kd] (gathered by token) or h [rows, Kd]
    int64_t lda;              // elements per activation row
    bool gather;              // true: row r reads activation row pair_of_row[r] / topk
    const int32_t* pair_of_row;
    int topk;
    const float* a_scale;     // FP8: [rows or T, Kd/128] activation scales, else null
    const void* w;            // [E, Nw, Kd] expert weights
    const void* w_scale;      // FP8: FP32 [E, Nw/128, Kd/128]; MXFP4: E8M0 bytes [E, Nw, Kd/32]; else null
    bool w_scale_pow2;        // FP8: every block scale is a power of two (the LDS-tiled GEMMs
                              // then apply only its exponent, with no significand fold)
    int n_out;                // output columns (I for gate/up, H for down)
    int kd;                   // reduction length
    const int32_t* exp_cnt;   // [E]
    const int32_t* exp_off;   // [E+1]
    const int2* tiles;        // [max_tiles] (expert, tile of the expert)
    const int32_t* meta;      // meta[kMetaTiles], meta[kMetaActive]
    const int32_t* active;    // [E] experts with rows, ascending
    int max_tiles;            // grid bound for tile-driven kernels
    int group_m;              // prefill block order: row tiles per XCD group (2 or 4)
    int max_active;           // grid bound for expert-driven kernels
    int max_rows;             // bound on the rows of one expert (min(T, T*K))
    void* out;                // [rows, n_out]
    int64_t ldo;              // elements per output row
    // When non-null the launcher may split K (for a single weight set, whose GEMMs alone
    // have too few blocks to fill the chip; streaming kernels over blockIdx.z, tiled ones
    // over a flat block order); slice z then writes FP32 partial sums to
    // part + z * part_slice instead of out: rows
    // of n_out sums for down, of 2 n_out for gate/up (gate sums, then up sums; the SwiGLU
    // is applied after the reduction).  part_cap bounds the floats of all slices.  The
    // launcher returns the slice count.
    float* part;
    int64_t part_slice;
    int64_t part_cap;
    int k_slices;             // LDS-tiled GEMMs: K slices of a split launch (set by the launcher)
    int64_t a_rows;           // rows of the activation matrix a (bounds the buffer loads of
                              // the 128-byte-stage kernels; set by the launcher)
};
constexpr int kMaxKSplit = 16;

// K slices for a GEMM of a single weight set with `blocks` blocks (column blocks of the
// streaming kernels, tiles of the LDS-tiled ones) whose partial sums take `out_elems`
// floats per slice: doubled while the grid holds fewer than four blocks per CU, every
// slice stays a multiple of `step` (the kernel's widest K step) and the slices fit in
// `cap` floats.
inline int decode_k_split(int64_t blocks, int kd, int step, int64_t out_elems, int64_t cap) {
    int s = 1;
    while (s < kMaxKSplit && blocks * s < 1024 && kd % (2 * s * step) == 0 && 2 * s * out_elems <= cap) s *= 2;
    return s;
}

// gemm_f32.hip (plain FP32, one thread per output)
void launch_gemm_f32(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, int64_t rows,
                     const int32_t* ids);
// gemm_bf16_decode.hip / gemm_fp8.hip: few rows per expert, weight streaming
// These return the number of K slices written to g.part (1: the result is in g.out).
int launch_gemm_bf16_decode(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g);
int launch_gemm_fp8_decode(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g);
// gemm_mxfp4.hip: MXFP4 weights, E4M3 activations, weight streaming
int launch_gemm_mxfp4_decode(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g);
// gemm_prefill.hip: 256 x 256 LDS-tiled MFMA, BF16, FP8 or MXFP4 weights
enum class PrefillWeights { kBf16, kFp8, kMxfp4 };
constexpr int kMxfp4PrefillMaxKd = 8192;    // LDS holds a tile's weight scales
constexpr int kFp8PrefillMaxKd = 32768;     // LDS holds the K-block scale codes past 64 blocks
// Returns the number of K slices written to g.part (1: the result is in g.out), which
// prefill_k_split gives beforehand.  MXFP4 slices hold at most kMxfp4PrefillMaxKd of K.
int launch_gemm_prefill(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, PrefillWeights wt);
int prefill_k_split(GemmMode mode, const GroupedGemmArgs& g, PrefillWeights wt);
// gemm_wide.hip: the same GEMMs for BF16 or FP8 weights (FP8: K <= 8192) with 128-byte
// K stages
int launch_gemm_wide(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, bool fp8);
// gemm_wide_mx.hip: the same for MXFP4 weights with 128-value K stages, for K slices of at
// most 6144 (wide_mx_supported); ks = prefill_k_split(mode, g, kMxfp4)
bool wide_mx_supported(const GroupedGemmArgs& g, int ks);
int launch_gemm_wide_mx(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, int ks);

// elementwise.hip
void launch_combine(hipStream_t st, int64_t T, int H, int K, bool f32, const void* yperm,
                    const int32_t* row_of_pair, const float* w, void* y);
void launch_prenorm(hipStream_t st, int64_t T, int H, const uint16_t* h, const float* gain,
                    float eps, float* xhat32, uint16_t* x_bf16, uint8_t* x_fp8, float* x_scale);
void launch_quant_rows_fp8(hipStream_t st, int64_t rows, int cols, bool src_bf16,
                           const void* src, uint8_t* q, float* scale);
void launch_post_residual(hipStream_t st, int64_t T, int H, int K, const uint16_t* yperm,
                          const int32_t* row_of_pair, const float* w, const float* gain,
                          float eps, float c1, float c2, uint16_t* h, uint16_t* moe_out);
// out[i] = BF16(part[0][i] + part[1][i] + ... + part[S-1][i]) for i < n (n % 8 == 0)
void launch_splitk_reduce(hipStream_t st, int S, int64_t n, int64_t slice, const float* part, uint16_t* out);
// h[r, c] = BF16(SiLU(sum_z part[z][r][c]) * sum_z part[z][r][n + c]) for r < rows, c < n
// (n % 8 == 0; part rows of 2n floats)
void launch_splitk_swiglu(hipStream_t st, int S, int64_t rows, int n, int64_t slice, const float* part,
                          uint16_t* h);
// Routing tables of a single weight set applied to every token (the dense MLP): one
// "expert" 0 holding rows 0..T-1 in token order, unit combine weights.
void launch_dense_setup(hipStream_t st, int64_t T, int BM, int32_t* ids, int32_t* exp_cnt, int32_t* exp_off,
                        int2* tiles, int32_t* meta, int32_t* active, int32_t* row_of_pair, int32_t* pair_of_row,
                        float* wts);

}  // namespace beam
