// BF16 grouped expert GEMMs on MFMA (gfx950), FP32 accumulation.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
// Rows r are the token->expert pairs sorted by expert, so each expert's rows are one
// contiguous range [exp_off[e], exp_off[e] + exp_cnt[e]).
//
// Two shapes:
//  * decode  (few rows per expert): the GEMM is a weight stream.  One block per
//    (active expert, 64 output columns); each wave streams 16 weight rows (32 for
//    gate/up) straight from HBM into MFMA B operands with deep unrolling, and the
//    expert's <= 16 activation rows ride along as the A operand (rows beyond the
//    expert's count issue no loads).  v_mfma_f32_16x16x32_bf16.
//  * prefill (many rows per expert): 128 x 128 output tiles from a device-built tile
//    list, 4 waves each owning 64 x 64 as 2 x 2 v_mfma_f32_32x32x16_bf16 tiles, K
//    staged through LDS 64 at a time with the next K-slab prefetched into registers.
//    For gate/up the 128 B-rows are 64 gate + 64 up rows of the same columns, so the
//    gate and up accumulators of one output land in the same lane and the SwiGLU is
//    applied in registers.
#include "common.cuh"
#include "kernels.h"

namespace beam {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------
// decode: weight streaming
// ---------------------------------------------------------------------------
template <int MODE, bool GATHER, int U>
__global__ __launch_bounds__(256) void gemm_bf16_decode(GroupedGemmArgs g) {
    const int slot = blockIdx.y;
    if (slot >= g.meta[kMetaActive]) return;
    const int e = g.active[slot];
    const int rows = g.exp_cnt[e], row0 = g.exp_off[e];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * 4 + wave) * 16;
    if (n0 >= g.n_out) return;
    const int ln = lane & 15, lq = lane >> 4;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const uint16_t* wp = static_cast<const uint16_t*>(g.w) +
                         (static_cast<int64_t>(e) * nw + n0 + ln) * g.kd + lq * 8;
    const uint16_t* wu = wp + static_cast<int64_t>(g.n_out) * g.kd;
    uint16_t* out = static_cast<uint16_t*>(g.out);

    for (int m0 = 0; m0 < rows; m0 += 16) {
        const int m = m0 + ln;
        const bool mv = m < rows;
        const int mr = mv ? m : rows - 1;
        const int64_t arow = GATHER ? g.pair_of_row[row0 + mr] / g.topk : static_cast<int64_t>(row0 + mr);
        const uint16_t* ap = static_cast<const uint16_t*>(g.a) + arow * g.lda + lq * 8;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < g.kd; k += 32 * U) {
            u32x4 b0[U], b1[U], a[U];
#pragma unroll
            for (int u = 0; u < U; ++u) b0[u] = *reinterpret_cast<const u32x4*>(wp + k + u * 32);
            if (MODE == kGateUp) {
#pragma unroll
                for (int u = 0; u < U; ++u) b1[u] = *reinterpret_cast<const u32x4*>(wu + k + u * 32);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                a[u] = u32x4{0u, 0u, 0u, 0u};
                if (mv) a[u] = *reinterpret_cast<const u32x4*>(ap + k + u * 32);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(b0[u]), acc0, 0, 0, 0);
                if (MODE == kGateUp)
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(b1[u]), acc1, 0, 0, 0);
            }
        }
        // C[m = lq*4 + i][n = ln]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = m0 + lq * 4 + i;
            if (mm >= rows) continue;
            const float v = (MODE == kGateUp) ? silu(acc0[i]) * acc1[i] : acc0[i];
            out[static_cast<int64_t>(row0 + mm) * g.ldo + n0 + ln] = f32_to_bf16_bits(v);
        }
    }
}

// ---------------------------------------------------------------------------
// prefill: LDS-tiled MFMA
// ---------------------------------------------------------------------------
template <int MODE, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_prefill(GroupedGemmArgs g) {
    constexpr int BM = kPrefillBM, BN = 128, BK = 64, LDK = BK + 8;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];
    constexpr int NCOL = (MODE == kGateUp) ? BN / 2 : BN;   // output columns per tile
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

    const uint16_t* ap[4];
    const uint16_t* bp[4];
    const int kc = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + i * 32;
        const int rr = min(r, rows - 1);
        const int64_t arow = GATHER ? g.pair_of_row[row0 + rr] / g.topk : static_cast<int64_t>(row0 + rr);
        ap[i] = static_cast<const uint16_t*>(g.a) + arow * g.lda + kc;
        int64_t wrow;
        if (MODE == kGateUp) wrow = (r < BN / 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        else wrow = c0 + r;
        bp[i] = static_cast<const uint16_t*>(g.w) + (static_cast<int64_t>(e) * nw + wrow) * g.kd + kc;
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
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[2], bfm[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                af[mi] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + mi * 32 + l32) * LDK + ks * 16 + lh * 8]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int brow = (MODE == kGateUp) ? (ni == 0 ? wn * 32 : BN / 2 + wn * 32) : wn * 64 + ni * 32;
                bfm[ni] = *reinterpret_cast<const bf16x8*>(&Bs[(brow + l32) * LDK + ks * 16 + lh * 8]);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfm[ni], acc[mi][ni], 0, 0, 0);
        }
    }
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * 64 + mi * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            if (m >= rows) continue;
            uint16_t* orow = out + static_cast<int64_t>(row0 + m) * g.ldo;
            if (MODE == kGateUp) {
                orow[c0 + wn * 32 + l32] = f32_to_bf16_bits(silu(acc[mi][0][i]) * acc[mi][1][i]);
            } else {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    orow[c0 + wn * 64 + ni * 32 + l32] = f32_to_bf16_bits(acc[mi][ni][i]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
void launch_gemm_bf16_decode(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g) {
    if (g.max_active == 0) return;
    dim3 grid((g.n_out + 63) / 64, g.max_active);
    const bool u8 = (g.kd % 256) == 0;
#define BEAM_DEC(M, GA, U) gemm_bf16_decode<M, GA, U><<<grid, 256, 0, st>>>(g)
    if (mode == kGateUp) {
        if (g.gather) { if (u8) BEAM_DEC(kGateUp, true, 8); else BEAM_DEC(kGateUp, true, 1); }
        else          { if (u8) BEAM_DEC(kGateUp, false, 8); else BEAM_DEC(kGateUp, false, 1); }
    } else {
        if (g.gather) { if (u8) BEAM_DEC(kDown, true, 8); else BEAM_DEC(kDown, true, 1); }
        else          { if (u8) BEAM_DEC(kDown, false, 8); else BEAM_DEC(kDown, false, 1); }
    }
#undef BEAM_DEC
}

void launch_gemm_bf16_prefill(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g) {
    if (g.max_tiles == 0) return;
    const int ncol = (mode == kGateUp) ? 64 : 128;
    const int blocks = g.max_tiles * (g.n_out / ncol);
    if (mode == kGateUp) {
        if (g.gather) gemm_bf16_prefill<kGateUp, true><<<blocks, 256, 0, st>>>(g);
        else gemm_bf16_prefill<kGateUp, false><<<blocks, 256, 0, st>>>(g);
    } else {
        if (g.gather) gemm_bf16_prefill<kDown, true><<<blocks, 256, 0, st>>>(g);
        else gemm_bf16_prefill<kDown, false><<<blocks, 256, 0, st>>>(g);
    }
}

}  // namespace beam
