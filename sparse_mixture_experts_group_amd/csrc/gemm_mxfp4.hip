// MXFP4 expert weights (OCP Microscaling Formats v1.0: FP4 E2M1 elements, one E8M0
// scale per 32 consecutive values along K) with E4M3 activations (one FP32 scale per
// row), for few rows per expert (decode): the grouped GEMM is a weight stream, as in the
// BF16 and FP8 streaming kernels, on v_mfma_scale_f32_16x16x128_f8f6f4 with an FP4 B
// operand.  The matrix core applies each weight block's E8M0 scale itself (one scale
// byte per lane), so the accumulation runs straight through K in FP32; the row scale of
// the activations is applied in the epilogue.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
//
// Operand layout of the 16x16x128 f8f6f4 MFMA with FP8 A and FP4 B (measured on gfx950):
// lane l = 16 q + c of the FP4 operand holds column c, K values 32 q .. 32 q + 31 (16
// bytes, element 2j in the low nibble of byte j), and its scale byte covers exactly those
// 32 values -- one MX block; the FP8 operand lane l = 16 q + r pairs with it when it holds
// row r, K values 16 q .. 16 q + 15 in bytes 0-15 and 64 + 16 q .. 64 + 16 q + 15 in
// bytes 16-31.
#include "common.cuh"
#include "kernels.h"

namespace beam {

namespace {
constexpr int kUnitScale = 0x7f;      // E8M0 code of 2^0
constexpr int kMxfp4Streams = 2;      // 16-row weight streams per wave
constexpr int kMxfp4U = 8;            // 128-wide K blocks per iteration

__device__ __forceinline__ i32x8 join_a(u32x4 lo, u32x4 hi) {
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ i32x8 fp4_operand(u32x4 v) {
    i32x8 r;
    r[0] = v[0]; r[1] = v[1]; r[2] = v[2]; r[3] = v[3];
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

__device__ __forceinline__ f32x4 mfma_a8w4(i32x8 a, i32x8 b, int scale_b, f32x4 c) {
    // format codes: A 0 = FP8 E4M3, B 4 = FP4 E2M1
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, kUnitScale, 0, scale_b);
}
}  // namespace

// One block per (active expert, 64 NS/2 output columns for gate/up, 64 NS for down);
// each wave streams NS groups of 16 weight rows (gate/up: NS/2 pairs of 16 gate + 16 up
// rows; down: NS x 16 consecutive rows) with U 128-wide K blocks of loads in flight, and
// the expert's activation rows ride along as A, 16 R per pass.
template <int MODE, bool GATHER, int U, int R, int NS>
__global__ __launch_bounds__(256) void gemm_mxfp4_decode(GroupedGemmArgs g) {
    const int slot = blockIdx.y;
    if (slot >= g.meta[kMetaActive]) return;
    const int e = g.active[slot];
    const int rows = g.exp_cnt[e], row0 = g.exp_off[e];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr int WC = (MODE == kGateUp) ? 8 * NS : 16 * NS;     // output columns per wave
    const int n0 = (blockIdx.x * 4 + wave) * WC;
    if (n0 >= g.n_out) return;
    const int ln = lane & 15, lq = lane >> 4;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const int64_t wrow_b = g.kd / 2, srow_b = g.kd / 32;       // bytes per weight / scale row
    const uint8_t* w = static_cast<const uint8_t*>(g.w);
    const uint8_t* sc = static_cast<const uint8_t*>(g.w_scale);      // E8M0 codes
    const uint8_t* wp[NS];
    const uint8_t* sp[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        // gate/up: stream 2j = gate rows of columns n0 + 16 j, 2j + 1 = their up rows
        const int64_t rr = (MODE == kGateUp)
            ? static_cast<int64_t>(e) * nw + n0 + 16 * (t >> 1) + ln + ((t & 1) ? g.n_out : 0)
            : static_cast<int64_t>(e) * nw + n0 + 16 * t + ln;
        wp[t] = w + rr * wrow_b + lq * 16;
        sp[t] = sc + rr * srow_b;
    }
    uint16_t* out = static_cast<uint16_t*>(g.out);
    // this block's K slice (the GEMMs of a single weight set split K over blockIdx.z)
    const int klen = g.kd / static_cast<int>(gridDim.z);
    const int kbeg = static_cast<int>(blockIdx.z) * klen;

    for (int m0 = 0; m0 < rows; m0 += 16 * R) {
        bool mv[R];
        const uint8_t* ap[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = m0 + 16 * r + ln;
            mv[r] = m < rows;
            const int mr = mv[r] ? m : rows - 1;
            const int64_t arow = GATHER ? g.pair_of_row[row0 + mr] / g.topk : static_cast<int64_t>(row0 + mr);
            ap[r] = static_cast<const uint8_t*>(g.a) + arow * g.lda + lq * 16;
        }
        f32x4 acc[R][NS];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NS; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k = kbeg; k < kbeg + klen; k += 128 * U) {
            u32x4 b[NS][U], a[R][U][2];
            // E8M0 scales of blocks k/32 + 4u + lq: byte lq of dword u of 4U bytes
            uint32_t s[NS][U];
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                if constexpr (U % 4 == 0) {
#pragma unroll
                    for (int v = 0; v < U / 4; ++v) {
                        const u32x4 sv = *reinterpret_cast<const u32x4*>(sp[t] + k / 32 + 16 * v);
#pragma unroll
                        for (int u = 0; u < 4; ++u) s[t][4 * v + u] = sv[u];
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) s[t][u] = *reinterpret_cast<const uint32_t*>(sp[t] + k / 32 + 4 * u);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) b[t][u] = *reinterpret_cast<const u32x4*>(wp[t] + (k + 128 * u) / 2);
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    a[r][u][0] = u32x4{0u, 0u, 0u, 0u};
                    a[r][u][1] = u32x4{0u, 0u, 0u, 0u};
                    if (mv[r]) {
                        a[r][u][0] = *reinterpret_cast<const u32x4*>(ap[r] + k + 128 * u);
                        a[r][u][1] = *reinterpret_cast<const u32x4*>(ap[r] + k + 128 * u + 64);
                    }
                }
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int t = 0; t < NS; ++t) {
                    const int scb = static_cast<int>((s[t][u] >> (8 * lq)) & 0xffu);
                    const i32x8 bb = fp4_operand(b[t][u]);
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[r][t] = mfma_a8w4(join_a(a[r][u][0], a[r][u][1]), bb, scb, acc[r][t]);
                }
            }
        }
        // C[m = lq*4 + i][n = ln] of row tile r
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = m0 + 16 * r + lq * 4 + i;
                if (mm >= rows) continue;
                const int64_t ar = GATHER ? g.pair_of_row[row0 + mm] / g.topk : static_cast<int64_t>(row0 + mm);
                const float sa = g.a_scale[ar];
                uint16_t* orow = out + static_cast<int64_t>(row0 + mm) * g.ldo + n0 + ln;
                if (MODE == kGateUp && gridDim.z > 1) {
                    // FP32 partial sums: gate then up sums (SwiGLU after the reduction)
                    float* prow = g.part + blockIdx.z * g.part_slice + static_cast<int64_t>(row0 + mm) * 2 * g.n_out + n0 + ln;
#pragma unroll
                    for (int j = 0; j < NS / 2; ++j) {
                        prow[16 * j] = acc[r][2 * j][i] * sa;
                        prow[g.n_out + 16 * j] = acc[r][2 * j + 1][i] * sa;
                    }
                } else if (MODE == kGateUp) {
#pragma unroll
                    for (int j = 0; j < NS / 2; ++j)
                        orow[16 * j] = f32_to_bf16_bits(silu(acc[r][2 * j][i] * sa) * (acc[r][2 * j + 1][i] * sa));
                } else if (gridDim.z > 1) {
                    float* prow = g.part + blockIdx.z * g.part_slice + static_cast<int64_t>(row0 + mm) * g.ldo + n0 + ln;
#pragma unroll
                    for (int t = 0; t < NS; ++t) prow[16 * t] = acc[r][t][i] * sa;
                } else {
#pragma unroll
                    for (int t = 0; t < NS; ++t) orow[16 * t] = f32_to_bf16_bits(acc[r][t][i] * sa);
                }
            }
    }
}

int launch_gemm_mxfp4_decode(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g) {
    if (g.max_active == 0) return 1;
    constexpr int NS = kMxfp4Streams;
    const int cols_per_block = 4 * ((mode == kGateUp) ? 8 * NS : 16 * NS);   // n_out: multiple of it
    const int nx = (g.n_out + cols_per_block - 1) / cols_per_block;
    const int64_t out_elems = static_cast<int64_t>(g.max_rows) * g.n_out * (mode == kGateUp ? 2 : 1);
    const int ks = g.part ? decode_k_split(static_cast<int64_t>(nx) * g.max_active, g.kd, 512, out_elems, g.part_cap) : 1;
    dim3 grid(nx, g.max_active, ks);
    // K blocks of 128 per iteration: as many as divide the slice
    const int klen = g.kd / ks;
    const int u = (klen % (128 * kMxfp4U) == 0) ? kMxfp4U : ((klen % 512 == 0) ? 4 : 1);
    const bool r2 = g.max_rows > 16;      // an expert can hold more than 16 rows
#define BEAM_DEC_U(M, GA, U) \
    do { if (r2) gemm_mxfp4_decode<M, GA, U, 2, NS><<<grid, 256, 0, st>>>(g); \
         else gemm_mxfp4_decode<M, GA, U, 1, NS><<<grid, 256, 0, st>>>(g); } while (0)
#define BEAM_DEC(M, GA) \
    do { if (u == kMxfp4U) BEAM_DEC_U(M, GA, kMxfp4U); else if (u == 4) BEAM_DEC_U(M, GA, 4); \
         else BEAM_DEC_U(M, GA, 1); } while (0)
    if (mode == kGateUp) {
        if (g.gather) BEAM_DEC(kGateUp, true);
        else BEAM_DEC(kGateUp, false);
    } else {
        if (g.gather) BEAM_DEC(kDown, true);
        else BEAM_DEC(kDown, false);
    }
#undef BEAM_DEC_U
#undef BEAM_DEC
    return ks;
}

}  // namespace beam
