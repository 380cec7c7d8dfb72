// FP8 (OCP E4M3FN) grouped expert GEMMs on the gfx950 f8f6f4 MFMA, FP32 accumulation.
//
// Weights carry one FP32 scale per 128 x 128 tile (value = code * scale); activations
// are quantised on the GPU with one FP32 scale per row (amax / 448).  The reduction is
// split into 128-wide K blocks, one weight-scale block each: the block's partial
// product is formed on the matrix core with unit hardware scales and folded into the
// FP32 accumulator with one fma by the (wave-uniform) weight scale; the row scale is
// applied once in the epilogue.  Same two shapes and the same SwiGLU fusion as the
// BF16 kernels (decode: weight streaming with v_mfma_scale_f32_16x16x128_f8f6f4;
// prefill: 128 x 128 LDS tiles with v_mfma_scale_f32_32x32x64_f8f6f4).
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

__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kUnitScale, 0, kUnitScale);
}
}  // namespace

// ---------------------------------------------------------------------------
// decode: weight streaming, 16 rows x 16 columns per wave
// ---------------------------------------------------------------------------
template <int MODE, bool GATHER, int U>
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
    const float* swg = g.w_scale + (static_cast<int64_t>(e) * (nw / 128) + n0 / 128) * kb_n;
    const float* swu = g.w_scale + (static_cast<int64_t>(e) * (nw / 128) + (g.n_out + n0) / 128) * kb_n;
    uint16_t* out = static_cast<uint16_t*>(g.out);

    for (int m0 = 0; m0 < rows; m0 += 16) {
        const int m = m0 + ln;
        const bool mv = m < rows;
        const int mr = mv ? m : rows - 1;
        const int64_t arow = GATHER ? g.pair_of_row[row0 + mr] / g.topk : static_cast<int64_t>(row0 + mr);
        const uint8_t* ap = static_cast<const uint8_t*>(g.a) + arow * g.lda + lq * 32;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < g.kd; k += 128 * U) {
            u32x4 b0[U][2], b1[U][2], a[U][2];
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
            for (int u = 0; u < U; ++u) {
                a[u][0] = u32x4{0u, 0u, 0u, 0u};
                a[u][1] = u32x4{0u, 0u, 0u, 0u};
                if (mv) {
                    a[u][0] = *reinterpret_cast<const u32x4*>(ap + k + u * 128);
                    a[u][1] = *reinterpret_cast<const u32x4*>(ap + k + u * 128 + 16);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kb = k / 128 + u;
                const i32x8 av = join(a[u][0], a[u][1]);
                const f32x4 t0 = mfma16_fp8(av, join(b0[u][0], b0[u][1]));
                const float s0 = swg[kb];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc0[i] = fmaf(t0[i], s0, acc0[i]);
                if (MODE == kGateUp) {
                    const f32x4 t1 = mfma16_fp8(av, join(b1[u][0], b1[u][1]));
                    const float s1 = swu[kb];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc1[i] = fmaf(t1[i], s1, acc1[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = m0 + lq * 4 + i;
            if (mm >= rows) continue;
            const int64_t ar = GATHER ? g.pair_of_row[row0 + mm] / g.topk : static_cast<int64_t>(row0 + mm);
            const float sa = g.a_scale[ar];
            const float v = (MODE == kGateUp) ? silu(acc0[i] * sa) * (acc1[i] * sa) : acc0[i] * sa;
            out[static_cast<int64_t>(row0 + mm) * g.ldo + n0 + ln] = f32_to_bf16_bits(v);
        }
    }
}

// ---------------------------------------------------------------------------
// prefill: 128 x 128 tiles, K blocks of 128 bytes staged through LDS
// ---------------------------------------------------------------------------
template <int MODE, bool GATHER>
__global__ __launch_bounds__(256) void gemm_fp8_prefill(GroupedGemmArgs g) {
    constexpr int BM = kPrefillBM, BN = 128, BK = 128, LDK = BK + 16;
    __shared__ __attribute__((aligned(16))) uint8_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * LDK];
    constexpr int NCOL = (MODE == kGateUp) ? BN / 2 : BN;
    const int n_tiles_n = g.n_out / NCOL;
    const int tile = blockIdx.x / n_tiles_n, nt = blockIdx.x % n_tiles_n;
    if (tile >= g.meta[kMetaTiles]) return;
    const int2 ti = g.tiles[tile];
    const int e = ti.x;
    const int rows = min(BM, g.exp_cnt[e] - ti.y);
    const int row0 = g.exp_off[e] + ti.y;
    const int c0 = nt * NCOL;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const int kb_n = g.kd / 128;

    const uint8_t* ap[4];
    const uint8_t* bp[4];
    const int kc = (tid & 7) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + i * 32;
        const int rr = min(r, rows - 1);
        const int64_t arow = GATHER ? g.pair_of_row[row0 + rr] / g.topk : static_cast<int64_t>(row0 + rr);
        ap[i] = static_cast<const uint8_t*>(g.a) + arow * g.lda + kc;
        int64_t wrow;
        if (MODE == kGateUp) wrow = (r < BN / 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        else wrow = c0 + r;
        bp[i] = static_cast<const uint8_t*>(g.w) + (static_cast<int64_t>(e) * nw + wrow) * g.kd + kc;
    }
    // weight-scale rows of this wave's two 32-column groups
    const float* sw[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        int64_t wrow;
        if (MODE == kGateUp) wrow = (ni == 0) ? c0 + wn * 32 : g.n_out + c0 + wn * 32;
        else wrow = c0 + wn * 64 + ni * 32;
        sw[ni] = g.w_scale + (static_cast<int64_t>(e) * (nw / 128) + wrow / 128) * kb_n;
    }

    u32x4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const u32x4*>(ap[i]);
        rb[i] = *reinterpret_cast<const u32x4*>(bp[i]);
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

    const int l32 = lane & 31, lh = lane >> 5;
    for (int k0 = 0; k0 < g.kd; k0 += BK) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + i * 32;
            *reinterpret_cast<u32x4*>(&As[r * LDK + kc]) = ra[i];
            *reinterpret_cast<u32x4*>(&Bs[r * LDK + kc]) = rb[i];
        }
        __syncthreads();
        if (k0 + BK < g.kd) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + k0 + BK);
                rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + k0 + BK);
            }
        }
        const int kb = k0 / 128;
        const float s0 = sw[0][kb], s1 = sw[1][kb];
        f32x16 tmp[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmp[mi][ni][i] = 0.0f;
#pragma unroll
        for (int hk = 0; hk < 2; ++hk) {
            i32x8 af[2], bfm[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const uint8_t* p = &As[(wm * 64 + mi * 32 + l32) * LDK + hk * 64 + lh * 32];
                af[mi] = join(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
            }
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int brow = (MODE == kGateUp) ? (ni == 0 ? wn * 32 : BN / 2 + wn * 32) : wn * 64 + ni * 32;
                const uint8_t* p = &Bs[(brow + l32) * LDK + hk * 64 + lh * 32];
                bfm[ni] = join(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) tmp[mi][ni] = mfma32_fp8(af[mi], bfm[ni], tmp[mi][ni]);
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc[mi][0][i] = fmaf(tmp[mi][0][i], s0, acc[mi][0][i]);
                acc[mi][1][i] = fmaf(tmp[mi][1][i], s1, acc[mi][1][i]);
            }
    }
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * 64 + mi * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            if (m >= rows) continue;
            const int64_t ar = GATHER ? g.pair_of_row[row0 + m] / g.topk : static_cast<int64_t>(row0 + m);
            const float sa = g.a_scale[ar];
            uint16_t* orow = out + static_cast<int64_t>(row0 + m) * g.ldo;
            if (MODE == kGateUp) {
                orow[c0 + wn * 32 + l32] = f32_to_bf16_bits(silu(acc[mi][0][i] * sa) * (acc[mi][1][i] * sa));
            } else {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    orow[c0 + wn * 64 + ni * 32 + l32] = f32_to_bf16_bits(acc[mi][ni][i] * sa);
            }
        }
    }
}

void launch_gemm_fp8(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, bool decode) {
    if (decode) {
        if (g.max_active == 0) return;
        dim3 grid((g.n_out + 63) / 64, g.max_active);
        const bool u4 = (g.kd % 512) == 0;
#define BEAM_DEC(M, GA, U) gemm_fp8_decode<M, GA, U><<<grid, 256, 0, st>>>(g)
        if (mode == kGateUp) {
            if (g.gather) { if (u4) BEAM_DEC(kGateUp, true, 4); else BEAM_DEC(kGateUp, true, 1); }
            else          { if (u4) BEAM_DEC(kGateUp, false, 4); else BEAM_DEC(kGateUp, false, 1); }
        } else {
            if (g.gather) { if (u4) BEAM_DEC(kDown, true, 4); else BEAM_DEC(kDown, true, 1); }
            else          { if (u4) BEAM_DEC(kDown, false, 4); else BEAM_DEC(kDown, false, 1); }
        }
#undef BEAM_DEC
        return;
    }
    if (g.max_tiles == 0) return;
    const int ncol = (mode == kGateUp) ? 64 : 128;
    const int blocks = g.max_tiles * (g.n_out / ncol);
    if (mode == kGateUp) {
        if (g.gather) gemm_fp8_prefill<kGateUp, true><<<blocks, 256, 0, st>>>(g);
        else gemm_fp8_prefill<kGateUp, false><<<blocks, 256, 0, st>>>(g);
    } else {
        if (g.gather) gemm_fp8_prefill<kDown, true><<<blocks, 256, 0, st>>>(g);
        else gemm_fp8_prefill<kDown, false><<<blocks, 256, 0, st>>>(g);
    }
}

}  // namespace beam
