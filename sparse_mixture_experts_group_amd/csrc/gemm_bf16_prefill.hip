// BF16 grouped expert GEMMs for many rows per expert (prefill-sized batches) on MFMA
// (gfx950), FP32 accumulation.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
// Rows r are the token->expert pairs sorted by expert, so each expert's rows are one
// contiguous range; the device-built tile list holds (expert, first row) per 256-row
// tile.  256 x 256 output tiles, 4 waves each owning 128 x 128 as 4 x 4
// v_mfma_f32_32x32x16_bf16 tiles, K staged through two LDS stages 64 at a time by
// direct global->LDS loads.  For gate/up the 256 B-rows are 128 gate + 128 up rows of
// the same columns, so the gate and up accumulators of one output land in the same lane
// and the SwiGLU is applied in registers.
#include "common.cuh"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// prefill: LDS-tiled MFMA, 256 x 256 block tile, 128 x 128 per wave
// ---------------------------------------------------------------------------
// Each wave owns a 128 x 128 output tile as 4 x 4 v_mfma_f32_32x32x16_bf16 tiles (256
// FP32 accumulators per lane), so a 16-wide K step reads 8 KB of LDS per wave for 16
// MFMAs.  K advances 64 at a time through two LDS stages filled by direct global->LDS
// loads (no register staging): the loads of K tile kt + 1 are issued when tile kt
// starts and waited for when it ends.
constexpr int kPfBK = 64;
constexpr int kPfStageBytes = 2 * kTileBytes;                  // A tile + B tile
constexpr size_t kPfLdsBytes = 2 * kPfStageBytes;

template <int MODE, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_prefill(GroupedGemmArgs g) {
    constexpr int BM = kPrefillBM, BN = 256, BK = kPfBK;
    static_assert(BM == kTileRows && BN == kTileRows && BK * 2 == kTileRowBytes, "tile geometry");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NCOL = (MODE == kGateUp) ? BN / 2 : BN;   // output columns per tile
    const int n_tiles_n = g.n_out / NCOL;
    int tile, nt;
    prefill_tile_of_block(n_tiles_n, tile, nt);
    if (tile >= g.meta[kMetaTiles]) return;
    const int2 ti = g.tiles[tile];
    const int e = ti.x;
    const int rows = min(BM, g.exp_cnt[e] - ti.y);
    const int row0 = g.exp_off[e] + ti.y;
    const int c0 = nt * NCOL;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;

    // Direct-to-LDS assignment: wave w moves rows w*64 + 8 j + lane/8 (j = 0..7) of both
    // operands; lane i fetches the global chunk that belongs in LDS slot i % 8.
    const int lr = lane >> 3, ls = lane & 7;
    const uint8_t* ag[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = wave * 64 + j * 8 + lr;
        const int rr = min(r, rows - 1);
        const int64_t arow = GATHER ? g.pair_of_row[row0 + rr] / g.topk : static_cast<int64_t>(row0 + rr);
        ag[j] = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(g.a) + arow * g.lda) +
                ((ls ^ ((r >> 1) & 7)) << 4);
    }
    // B rows of wave w are affine in j (for gate/up, waves 0-1 move gate rows, 2-3 up rows)
    const uint8_t* bg;
    {
        const int r = wave * 64 + lr;
        int64_t wrow;
        if (MODE == kGateUp) wrow = (wave < 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        else wrow = c0 + r;
        bg = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(g.w) + (static_cast<int64_t>(e) * nw + wrow) * g.kd);
    }
    const int64_t bstep = 8 * static_cast<int64_t>(g.kd) * 2;      // bytes between j and j + 1
    // swizzle of row r = w*64 + 8 j + lr: ((r >> 1) & 7) = 4 (j & 1) + (lr >> 1)
    const int boff_lane[2] = {(ls ^ (lr >> 1)) << 4, (ls ^ (4 + (lr >> 1))) << 4};
    auto dma = [&](int stage, int k0) {
        uint8_t* As = smem + stage * kPfStageBytes;
        uint8_t* Bs = As + kTileBytes;
        const int kb = k0 * 2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __builtin_amdgcn_global_load_lds(ag[j] + kb, As + (wave * 64 + j * 8) * kTileRowBytes, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(bg + j * bstep + kb + boff_lane[j & 1], Bs + (wave * 64 + j * 8) * kTileRowBytes,
                                             16, 0, 0);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

    const int l32 = lane & 31, lh = lane >> 5;
    int arow_l[4], brow_l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        arow_l[i] = wm * 128 + i * 32 + l32;
        brow_l[i] = (MODE == kGateUp) ? ((i < 2) ? wn * 64 + i * 32 : BN / 2 + wn * 64 + (i - 2) * 32) + l32
                                      : wn * 128 + i * 32 + l32;
    }
    bf16x8 fa[2][4], fb[2][4];     // fragments, double-buffered over K steps
    auto load_frags = [&](int buf, int stage, int ks) {
        const uint8_t* As = smem + stage * kPfStageBytes;
        const uint8_t* Bs = As + kTileBytes;
        const int c = ks * 2 + lh;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            fa[buf][mi] = *reinterpret_cast<const bf16x8*>(As + tile_offset(arow_l[mi], c));
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            fb[buf][ni] = *reinterpret_cast<const bf16x8*>(Bs + tile_offset(brow_l[ni], c));
    };

    const int nk = g.kd / BK;
    dma(0, 0);
    wait_lds_dma();
    __syncthreads();
    load_frags(0, 0, 0);
    // The loop body is branch-free so the scheduling fences apply to whole K steps: the
    // memory operations of a step are issued first, then its 16 independent MFMAs, and
    // nothing is hoisted across steps.  The last iteration re-loads the last slab into
    // the idle stage (clamped index), which nothing reads.
    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt & 1;
        __builtin_amdgcn_sched_barrier(0);
        dma(stage ^ 1, min(kt + 1, nk - 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < BK / 16) load_frags(cur ^ 1, stage, ks + 1);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][mi], fb[cur][ni], acc[mi][ni], 0, 0, 0);
            if (ks + 1 < BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS reads first
            __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);                        // then MFMAs
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_lds_dma();
        __syncthreads();
        load_frags(0, stage ^ 1, 0);
    }

    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * 128 + mi * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            if (m >= rows) continue;
            uint16_t* orow = out + static_cast<int64_t>(row0 + m) * g.ldo;
            if (MODE == kGateUp) {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    orow[c0 + wn * 64 + ni * 32 + l32] = f32_to_bf16_bits(silu(acc[mi][ni][i]) * acc[mi][ni + 2][i]);
            } else {
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    orow[c0 + wn * 128 + ni * 32 + l32] = f32_to_bf16_bits(acc[mi][ni][i]);
            }
        }
    }
}

template <int MODE, bool GATHER>
void launch_prefill_inst(hipStream_t st, const GroupedGemmArgs& g, int blocks) {
    static bool attr_set = false;     // the LDS opt-in is per kernel, set on first use
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_prefill<MODE, GATHER>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kPfLdsBytes));
        attr_set = true;
    }
    gemm_bf16_prefill<MODE, GATHER><<<blocks, 256, kPfLdsBytes, st>>>(g);
}

void launch_gemm_bf16_prefill(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g) {
    if (g.max_tiles == 0) return;
    const int ncol = (mode == kGateUp) ? 128 : 256;
    const int blocks = (g.max_tiles * (g.n_out / ncol) + 255) / 256 * 256;   // whole XCD chunks
    if (mode == kGateUp) {
        if (g.gather) launch_prefill_inst<kGateUp, true>(st, g, blocks);
        else launch_prefill_inst<kGateUp, false>(st, g, blocks);
    } else {
        if (g.gather) launch_prefill_inst<kDown, true>(st, g, blocks);
        else launch_prefill_inst<kDown, false>(st, g, blocks);
    }
}

}  // namespace beam
