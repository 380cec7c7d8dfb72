// BF16 grouped expert GEMMs for few rows per expert (decode-sized batches): the GEMM is
// a weight stream.  MFMA (gfx950) with FP32 accumulation.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
// Rows r are the token->expert pairs sorted by expert, so each expert's rows are one
// contiguous range [exp_off[e], exp_off[e] + exp_cnt[e]).
//
// One block per (active expert, 64 output columns for gate/up, 128 for down, K slice);
// each wave streams 32 weight rows (16 gate + 16 up, or 32 down rows) straight from HBM
// into MFMA B operands with deep unrolling, and the expert's activation rows ride along
// as the A operand, 16 or 32 at a time (rows beyond the expert's count issue no loads).
// The GEMMs of a single weight set split K over blockIdx.z (FP32 partial sums).
// v_mfma_f32_16x16x32_bf16.
#include "common.cuh"
#include "kernels.h"

namespace beam {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------
// decode: weight streaming
// ---------------------------------------------------------------------------
template <int MODE, bool GATHER, int U, int R>
__global__ __launch_bounds__(256) void gemm_bf16_decode(GroupedGemmArgs g) {
    const int slot = blockIdx.y;
    if (slot >= g.meta[kMetaActive]) return;
    const int e = g.active[slot];
    const int rows = g.exp_cnt[e], row0 = g.exp_off[e];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // gate/up: 16 output columns per wave, streams of their gate and up rows; down: 32
    // output columns per wave as two streams of 16 rows
    constexpr int WC = (MODE == kGateUp) ? 16 : 32;
    const int n0 = (blockIdx.x * 4 + wave) * WC;
    if (n0 >= g.n_out) return;
    const int ln = lane & 15, lq = lane >> 4;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const uint16_t* wp = static_cast<const uint16_t*>(g.w) +
                         (static_cast<int64_t>(e) * nw + n0 + ln) * g.kd + lq * 8;
    const uint16_t* wu = wp + static_cast<int64_t>(MODE == kGateUp ? g.n_out : 16) * g.kd;
    uint16_t* out = static_cast<uint16_t*>(g.out);
    const int klen = g.kd / static_cast<int>(gridDim.z);          // this block's K slice
    const int kbeg = static_cast<int>(blockIdx.z) * klen;

    // R row tiles of 16 per pass: each weight fragment feeds R MFMAs, so experts with up
    // to 16 R rows stream their weights once.
    for (int m0 = 0; m0 < rows; m0 += 16 * R) {
        bool mv[R];
        const uint16_t* ap[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = m0 + 16 * r + ln;
            mv[r] = m < rows;
            const int mr = mv[r] ? m : rows - 1;
            const int64_t arow = GATHER ? g.pair_of_row[row0 + mr] / g.topk : static_cast<int64_t>(row0 + mr);
            ap[r] = static_cast<const uint16_t*>(g.a) + arow * g.lda + lq * 8;
        }
        f32x4 acc0[R], acc1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) { acc0[r] = f32x4{0.f, 0.f, 0.f, 0.f}; acc1[r] = f32x4{0.f, 0.f, 0.f, 0.f}; }
        for (int k = kbeg; k < kbeg + klen; k += 32 * U) {
            u32x4 b0[U], b1[U], a[R][U];
#pragma unroll
            for (int u = 0; u < U; ++u) b0[u] = *reinterpret_cast<const u32x4*>(wp + k + u * 32);
#pragma unroll
            for (int u = 0; u < U; ++u) b1[u] = *reinterpret_cast<const u32x4*>(wu + k + u * 32);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    a[r][u] = u32x4{0u, 0u, 0u, 0u};
                    if (mv[r]) a[r][u] = *reinterpret_cast<const u32x4*>(ap[r] + k + u * 32);
                }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    acc0[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[r][u]), as_bf16x8(b0[u]), acc0[r], 0, 0, 0);
                    acc1[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[r][u]), as_bf16x8(b1[u]), acc1[r], 0, 0, 0);
                }
        }
        // C[m = lq*4 + i][n = ln] of row tile r
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = m0 + 16 * r + lq * 4 + i;
                if (mm >= rows) continue;
                uint16_t* orow = out + static_cast<int64_t>(row0 + mm) * g.ldo + n0 + ln;
                if (MODE == kGateUp && gridDim.z > 1) {
                    float* prow = g.part + blockIdx.z * g.part_slice + static_cast<int64_t>(row0 + mm) * 2 * g.n_out + n0 + ln;
                    prow[0] = acc0[r][i];
                    prow[g.n_out] = acc1[r][i];
                } else if (MODE == kGateUp) {
                    orow[0] = f32_to_bf16_bits(silu(acc0[r][i]) * acc1[r][i]);
                } else if (gridDim.z > 1) {
                    float* prow = g.part + blockIdx.z * g.part_slice + static_cast<int64_t>(row0 + mm) * g.ldo + n0 + ln;
                    prow[0] = acc0[r][i];
                    prow[16] = acc1[r][i];
                } else {
                    orow[0] = f32_to_bf16_bits(acc0[r][i]);
                    orow[16] = f32_to_bf16_bits(acc1[r][i]);
                }
            }
    }
}

int launch_gemm_bf16_decode(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g) {
    if (g.max_active == 0) return 1;
    const int cols_per_block = (mode == kGateUp) ? 64 : 128;     // n_out is a multiple of 32
    const int nx = (g.n_out + cols_per_block - 1) / cols_per_block;
    const int64_t out_elems = static_cast<int64_t>(g.max_rows) * g.n_out * (mode == kGateUp ? 2 : 1);
    const int ks = g.part ? decode_k_split(static_cast<int64_t>(nx) * g.max_active, g.kd, 256, out_elems, g.part_cap) : 1;
    dim3 grid(nx, g.max_active, ks);
    const bool u8 = ((g.kd / ks) % 256) == 0;
    const bool r2 = g.max_rows > 16;      // an expert can hold more than 16 rows
#define BEAM_DEC(M, GA, U) \
    do { if (r2) gemm_bf16_decode<M, GA, U, 2><<<grid, 256, 0, st>>>(g); \
         else gemm_bf16_decode<M, GA, U, 1><<<grid, 256, 0, st>>>(g); } while (0)
    if (mode == kGateUp) {
        if (g.gather) { if (u8) BEAM_DEC(kGateUp, true, 8); else BEAM_DEC(kGateUp, true, 1); }
        else          { if (u8) BEAM_DEC(kGateUp, false, 8); else BEAM_DEC(kGateUp, false, 1); }
    } else {
        if (g.gather) { if (u8) BEAM_DEC(kDown, true, 8); else BEAM_DEC(kDown, true, 1); }
        else          { if (u8) BEAM_DEC(kDown, false, 8); else BEAM_DEC(kDown, false, 1); }
    }
#undef BEAM_DEC
    return ks;
}

}  // namespace beam
