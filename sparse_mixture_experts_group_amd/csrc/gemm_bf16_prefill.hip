// BF16 grouped expert GEMMs for many rows per expert (prefill-sized batches) on MFMA
// (gfx950), FP32 accumulation.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
// Rows r are the token->expert pairs sorted by expert, so each expert's rows are one
// contiguous range; the device-built tile list holds (expert, first row) per BM-row
// tile (BM = 256, or 128 when experts average fewer than ~192 rows).  BM x 256 output
// tiles, 4 waves each owning (BM/2) x 128 as (BM/64) x 4 v_mfma_f32_32x32x16_bf16
// tiles, K staged through two LDS stages 64 at a time by direct global->LDS loads.  For gate/up the 256 B-rows are 128 gate + 128 up rows of
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
template <int BM> constexpr int pf_stage_bytes() { return (BM + kTileRows) * kTileRowBytes; }   // A + B tiles
// LDS stages: 2 x 64 KB for 256-row tiles; 3 x 48 KB for 128-row tiles, whose GEMM is
// bound by streaming the weights and needs more bytes in flight per CU.
template <int BM> constexpr int pf_stages() { return BM == 256 ? 2 : 3; }
template <int BM> constexpr size_t pf_lds_bytes() { return pf_stages<BM>() * pf_stage_bytes<BM>(); }

// BM = 256: each wave owns 128 rows (4 MFMA row tiles); BM = 128: 64 rows (2 row tiles).
template <int MODE, bool GATHER, int BM>
__global__ __launch_bounds__(256) void gemm_bf16_prefill(GroupedGemmArgs g) {
    constexpr int BN = 256, BK = kPfBK, MI = BM / 64, WROWS = BM / 2;
    constexpr int kPfStageBytes = pf_stage_bytes<BM>();
    static_assert((BM == 256 || BM == 128) && BN == kTileRows && BK * 2 == kTileRowBytes, "tile geometry");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NCOL = (MODE == kGateUp) ? BN / 2 : BN;   // output columns per tile
    const int n_tiles_n = g.n_out / NCOL;
    int tile, nt;
    prefill_tile_of_block(n_tiles_n, BM == 256 ? 4 : 1, tile, nt);
    if (tile >= g.meta[kMetaTiles]) return;
    const int2 ti = g.tiles[tile];
    const int e = ti.x;
    const int rows = min(BM, g.exp_cnt[e] - ti.y);
    const int row0 = g.exp_off[e] + ti.y;
    const int c0 = nt * NCOL;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;

    // Direct-to-LDS assignment: wave w moves A rows w*BM/4 + 8 j + lane/8 (j < BM/32) and
    // B rows w*64 + 8 j + lane/8 (j < 8); lane i fetches the global chunk that belongs in
    // LDS slot i % 8.
    const int lr = lane >> 3, ls = lane & 7;
    constexpr int AJ = BM / 32;
    const uint8_t* ag[AJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
        const int r = wave * (BM / 4) + j * 8 + lr;
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
        uint8_t* Bs = As + BM * kTileRowBytes;
        const int kb = k0 * 2;
#pragma unroll
        for (int j = 0; j < AJ; ++j)
            lds_dma16(ag[j] + kb, As + (wave * (BM / 4) + j * 8) * kTileRowBytes);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            lds_dma16(bg + j * bstep + kb + boff_lane[j & 1], Bs + (wave * 64 + j * 8) * kTileRowBytes);
    };

    f32x16 acc[MI][4];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

    const int l32 = lane & 31, lh = lane >> 5;
    int arow_l[MI], brow_l[4];
#pragma unroll
    for (int i = 0; i < MI; ++i) arow_l[i] = wm * WROWS + i * 32 + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        brow_l[i] = (MODE == kGateUp) ? ((i < 2) ? wn * 64 + i * 32 : BN / 2 + wn * 64 + (i - 2) * 32) + l32
                                      : wn * 128 + i * 32 + l32;
    }
    // 32-row MFMA tiles of this wave that hold rows of the expert (wave-uniform): the
    // others (padding of an expert's last tile) skip their LDS reads and MFMAs.
    const int mvalid = __builtin_amdgcn_readfirstlane(min(MI, max(0, (rows - wm * WROWS + 31) / 32)));
    bf16x8 fa[2][MI], fb[2][4];     // fragments, double-buffered over K steps
    // The K loop is instantiated per count MV of live row tiles: each instance is
    // branch-free, and tiles past the expert's last row skip their LDS reads and MFMAs.
    auto k_loop = [&](auto mv_tag) {
        constexpr int MV = decltype(mv_tag)::value;
        auto load_frags = [&](int buf, int stage, int ks) {
            const uint8_t* As = smem + stage * kPfStageBytes;
            const uint8_t* Bs = As + BM * kTileRowBytes;
            const int c = ks * 2 + lh;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                if (mi < MV) fa[buf][mi] = *reinterpret_cast<const bf16x8*>(As + tile_offset(arow_l[mi], c));
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                fb[buf][ni] = *reinterpret_cast<const bf16x8*>(Bs + tile_offset(brow_l[ni], c));
        };

        // NST-stage pipeline: the loads of K tile kt + NST - 1 are issued when tile kt starts;
        // at the end of tile kt each wave waits until only the loads of the tiles after kt + 1
        // are outstanding (PER loads per tile), then the block synchronises.
        constexpr int NST = pf_stages<BM>();
        constexpr int PER = AJ + 8;
        const int nk = g.kd / BK;
#pragma unroll
        for (int s0 = 0; s0 < NST - 1; ++s0) dma(s0, min(s0, nk - 1) * BK);
        wait_lds_dma<(NST - 2) * PER>();
        lds_pipeline_barrier();
        load_frags(0, 0, 0);
        // The loop body is branch-free so the scheduling fences apply to whole K steps: the
        // memory operations of a step are issued first, then its independent MFMAs, and
        // nothing is hoisted across steps.  Past the end the slab index is clamped: the last
        // iterations re-load the last slab into stages that nothing reads any more.
        int stage = 0;
        for (int kt = 0; kt < nk; ++kt) {
            const int nstage = (stage + 1 == NST) ? 0 : stage + 1;
            const int lstage = (stage == 0) ? NST - 1 : stage - 1;   // = (kt + NST - 1) % NST
            __builtin_amdgcn_sched_barrier(0);
            dma(lstage, min(kt + NST - 1, nk - 1) * BK);
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int cur = ks & 1;
                __builtin_amdgcn_sched_barrier(0);
                if (ks + 1 < BK / 16) load_frags(cur ^ 1, stage, ks + 1);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) {
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][mi], fb[cur][ni], acc[mi][ni], 0, 0, 0);
                    }
                // DS reads first, then MFMAs (builtin arguments must be literal constants)
                if constexpr (MI == 4) {
                    if (ks + 1 < BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
                } else {
                    if (ks + 1 < BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_lds_dma<(NST - 2) * PER>();
            lds_pipeline_barrier();
            load_frags(0, nstage, 0);
            stage = nstage;
        }
    };
    dispatch_row_tiles<MI>(mvalid, k_loop);

    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * WROWS + mi * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
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

template <int MODE, bool GATHER, int BM>
void launch_prefill_inst(hipStream_t st, const GroupedGemmArgs& g, int blocks) {
    static bool attr_set = false;     // the LDS opt-in is per kernel, set on first use
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_prefill<MODE, GATHER, BM>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(pf_lds_bytes<BM>()));
        attr_set = true;
    }
    gemm_bf16_prefill<MODE, GATHER, BM><<<blocks, 256, pf_lds_bytes<BM>(), st>>>(g);
}

void launch_gemm_bf16_prefill(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g) {
    if (g.max_tiles == 0) return;
    const int ncol = (mode == kGateUp) ? 128 : 256;
    const int blocks = (g.max_tiles * (g.n_out / ncol) + 255) / 256 * 256;   // whole XCD chunks
    const bool small = g.bm == kPrefillBMMin;
    if (mode == kGateUp) {
        if (g.gather) {
            if (small) launch_prefill_inst<kGateUp, true, kPrefillBMMin>(st, g, blocks);
            else launch_prefill_inst<kGateUp, true, kPrefillBMMax>(st, g, blocks);
        } else {
            if (small) launch_prefill_inst<kGateUp, false, kPrefillBMMin>(st, g, blocks);
            else launch_prefill_inst<kGateUp, false, kPrefillBMMax>(st, g, blocks);
        }
    } else {
        if (g.gather) {
            if (small) launch_prefill_inst<kDown, true, kPrefillBMMin>(st, g, blocks);
            else launch_prefill_inst<kDown, true, kPrefillBMMax>(st, g, blocks);
        } else {
            if (small) launch_prefill_inst<kDown, false, kPrefillBMMin>(st, g, blocks);
            else launch_prefill_inst<kDown, false, kPrefillBMMax>(st, g, blocks);
        }
    }
}

}  // namespace beam
