// FP8 (OCP E4M3FN) grouped expert GEMMs for few rows per expert (decode) on the gfx950
// f8f6f4 MFMA, FP32 accumulation.
//
// Weights carry one FP32 scale per 128 x 128 tile (value = code * scale); activations
// are quantised on the GPU with one FP32 scale per row (amax / 448).  The reduction is
// split into 128-wide K blocks, one weight-scale block each: the block's partial
// product is formed on the matrix core with unit hardware scales and folded into the
// FP32 accumulator with one fma by the (wave-uniform) weight scale; the row scale is
// applied once in the epilogue.  Weight streaming with v_mfma_scale_f32_16x16x128_f8f6f4
// and the same SwiGLU fusion as the BF16 decode kernel.
#include "common.cuh"
#include "kernels.h"

namespace beam {

namespace {
constexpr int kUnitScale = 0x7f7f7f7f;   // E8M0 exponent 127 = 2^0 in every byte

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ f32x4 mfma16_fp8(i32x8 a, i32x8 b) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, kUnitScale, 0, kUnitScale);
}

}  // namespace

// ---------------------------------------------------------------------------
// decode: weight streaming, 16 columns per wave, 16 or 32 rows per pass
// ---------------------------------------------------------------------------
template <int MODE, bool GATHER, int U, int R>
__global__ __launch_bounds__(256) void gemm_fp8_decode(GroupedGemmArgs g) {
    const int slot = blockIdx.y;
    if (slot >= g.meta[kMetaActive]) return;
    const int e = g.active[slot];
    const int rows = g.exp_cnt[e], row0 = g.exp_off[e];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * 4 + wave) * 16;
    if (n0 >= g.n_out) return;
    const int ln = lane & 15, lq = lane >> 4;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const int kb_n = g.kd / 128;
    const uint8_t* wp = static_cast<const uint8_t*>(g.w) + (static_cast<int64_t>(e) * nw + n0 + ln) * g.kd + lq * 32;
    const uint8_t* wu = wp + static_cast<int64_t>(g.n_out) * g.kd;
    const float* wsc = static_cast<const float*>(g.w_scale);      // FP32 block scales
    const float* swg = wsc + (static_cast<int64_t>(e) * (nw / 128) + n0 / 128) * kb_n;
    const float* swu = wsc + (static_cast<int64_t>(e) * (nw / 128) + (g.n_out + n0) / 128) * kb_n;
    uint16_t* out = static_cast<uint16_t*>(g.out);
    // this block's K slice (the GEMMs of a single weight set split K over blockIdx.z)
    const int klen = g.kd / static_cast<int>(gridDim.z);
    const int kbeg = static_cast<int>(blockIdx.z) * klen;

    // R row tiles of 16 per pass: each weight fragment feeds R MFMAs, so experts with up
    // to 16 R rows stream their weights once.
    for (int m0 = 0; m0 < rows; m0 += 16 * R) {
        bool mv[R];
        const uint8_t* ap[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = m0 + 16 * r + ln;
            mv[r] = m < rows;
            const int mr = mv[r] ? m : rows - 1;
            const int64_t arow = GATHER ? g.pair_of_row[row0 + mr] / g.topk : static_cast<int64_t>(row0 + mr);
            ap[r] = static_cast<const uint8_t*>(g.a) + arow * g.lda + lq * 32;
        }
        f32x4 acc0[R], acc1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) { acc0[r] = f32x4{0.f, 0.f, 0.f, 0.f}; acc1[r] = f32x4{0.f, 0.f, 0.f, 0.f}; }
        for (int k = kbeg; k < kbeg + klen; k += 128 * U) {
            u32x4 b0[U][2], b1[U][2], a[R][U][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                b0[u][0] = *reinterpret_cast<const u32x4*>(wp + k + u * 128);
                b0[u][1] = *reinterpret_cast<const u32x4*>(wp + k + u * 128 + 16);
            }
            if (MODE == kGateUp) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    b1[u][0] = *reinterpret_cast<const u32x4*>(wu + k + u * 128);
                    b1[u][1] = *reinterpret_cast<const u32x4*>(wu + k + u * 128 + 16);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    a[r][u][0] = u32x4{0u, 0u, 0u, 0u};
                    a[r][u][1] = u32x4{0u, 0u, 0u, 0u};
                    if (mv[r]) {
                        a[r][u][0] = *reinterpret_cast<const u32x4*>(ap[r] + k + u * 128);
                        a[r][u][1] = *reinterpret_cast<const u32x4*>(ap[r] + k + u * 128 + 16);
                    }
                }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kb = k / 128 + u;
                const float s0 = swg[kb];
                const float s1 = (MODE == kGateUp) ? swu[kb] : 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const i32x8 av = join(a[r][u][0], a[r][u][1]);
                    const f32x4 t0 = mfma16_fp8(av, join(b0[u][0], b0[u][1]));
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc0[r][i] = fmaf(t0[i], s0, acc0[r][i]);
                    if (MODE == kGateUp) {
                        const f32x4 t1 = mfma16_fp8(av, join(b1[u][0], b1[u][1]));
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc1[r][i] = fmaf(t1[i], s1, acc1[r][i]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = m0 + 16 * r + lq * 4 + i;
                if (mm >= rows) continue;
                const int64_t ar = GATHER ? g.pair_of_row[row0 + mm] / g.topk : static_cast<int64_t>(row0 + mm);
                const float sa = g.a_scale[ar];
                if (gridDim.z > 1) {
                    // FP32 partial sums: gate then up sums for gate/up (SwiGLU after the reduction)
                    const int64_t o = static_cast<int64_t>(row0 + mm) * (MODE == kGateUp ? 2 * g.n_out : g.ldo) + n0 + ln;
                    float* pz = g.part + blockIdx.z * g.part_slice;
                    pz[o] = acc0[r][i] * sa;
                    if (MODE == kGateUp) pz[o + g.n_out] = acc1[r][i] * sa;
                    continue;
                }
                const float v = (MODE == kGateUp) ? silu(acc0[r][i] * sa) * (acc1[r][i] * sa) : acc0[r][i] * sa;
                out[static_cast<int64_t>(row0 + mm) * g.ldo + n0 + ln] = f32_to_bf16_bits(v);
            }
    }
}

int launch_gemm_fp8_decode(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g) {
    if (g.max_active == 0) return 1;
    const int nx = (g.n_out + 63) / 64;
    const int64_t out_elems = static_cast<int64_t>(g.max_rows) * g.n_out * (mode == kGateUp ? 2 : 1);
    const int ks = g.part ? decode_k_split(static_cast<int64_t>(nx) * g.max_active, g.kd, 512, out_elems, g.part_cap) : 1;
    dim3 grid(nx, g.max_active, ks);
    const bool u4 = ((g.kd / ks) % 512) == 0;
    const bool r2 = g.max_rows > 16;      // an expert can hold more than 16 rows
#define BEAM_DEC(M, GA, U) \
    do { if (r2) gemm_fp8_decode<M, GA, U, 2><<<grid, 256, 0, st>>>(g); \
         else gemm_fp8_decode<M, GA, U, 1><<<grid, 256, 0, st>>>(g); } while (0)
    if (mode == kGateUp) {
        if (g.gather) { if (u4) BEAM_DEC(kGateUp, true, 4); else BEAM_DEC(kGateUp, true, 1); }
        else          { if (u4) BEAM_DEC(kGateUp, false, 4); else BEAM_DEC(kGateUp, false, 1); }
    } else {
        if (g.gather) { if (u4) BEAM_DEC(kDown, true, 4); else BEAM_DEC(kDown, true, 1); }
        else          { if (u4) BEAM_DEC(kDown, false, 4); else BEAM_DEC(kDown, false, 1); }
    }
#undef BEAM_DEC
    return ks;
}

}  // namespace beam
