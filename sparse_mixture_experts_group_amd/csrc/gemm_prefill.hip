// Grouped expert GEMMs for many rows per expert (prefill-sized batches) on the gfx950
// matrix cores, FP32 accumulation, BF16 or FP8 (OCP E4M3FN) operands.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
// Rows r are the token->expert pairs sorted by expert, so each expert's rows are one
// contiguous range; the device-built tile list splits each expert's rows into
// ceil(rows / 256) tiles of whole 32-row blocks, as equal as possible.  256 x 256
// output tiles; 4 waves, each owning 128 x 128 as 4 x 4 MFMA tiles of 32 x 32
// (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4).  For gate/up the 256
// weight rows of a tile are 128 gate + 128 up rows of the same columns, so the gate and
// up accumulators of one output land in the same lane and the SwiGLU is applied in
// registers.
//
// FP8: weights carry one power-of-two scale per 128 x 128 block, which the f8f6f4 MFMA
// applies itself as the E8M0 scale of its B operand (the FP32 scale's exponent field is
// the E8M0 code), so the accumulation needs no per-block fold.  Activations carry one
// FP32 scale per row, applied in the epilogue.
#include "common.cuh"
#include "kernels.h"

namespace beam {

namespace {
constexpr int kUnitScale = 0x7f;                // E8M0 code of 2^0

// K advances 64 bytes per LDS stage (32 BF16 or 64 FP8 values); A (256 rows) and B
// (256 rows) take 32 KB per stage.
constexpr int kStageBytes = (kPrefillBM + 256) * kStageRowBytes;
constexpr int kStages = 4;
constexpr size_t kLdsBytes = kStages * kStageBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Fragments of one LDS stage for one wave: BF16 - two 16-wide K steps of 8 values per
// lane; FP8 - one 64-wide K step of 32 values per lane.
template <bool FP8> struct StageFrags;
template <> struct StageFrags<false> { bf16x8 a[2][4]; bf16x8 b[2][4]; };
template <> struct StageFrags<true> { i32x8 a[4]; i32x8 b[4]; };
}  // namespace

// Block work: one (256-row tile, column tile).  Wave (wm, wn) owns the 32-row MFMA
// tiles wm, wm + 2, wm + 4, wm + 6 (the padding rows of an expert's last tile are
// shared out evenly between the two wave rows) and 128 columns.
//
// Pipeline (kStages = 4 LDS stages, filled by direct global->LDS loads): iteration j
// waits until stage j + 1 has landed for every wave, then runs the MFMAs of stage j
// from registers while reading the fragments of stage j + 1 and loading stage j + 4
// into the slot of stage j, whose fragments were read in the previous iteration.  So
// three stages are in flight while one is computed.
template <int MODE, bool GATHER, bool FP8>
__global__ __launch_bounds__(256) void gemm_prefill(GroupedGemmArgs g) {
    constexpr int BM = kPrefillBM, BN = 256, MI = 4, NST = kStages;
    constexpr int EB = FP8 ? 1 : 2;                     // bytes per element
    constexpr int BK = kStageRowBytes / EB;             // K per stage
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NCOL = (MODE == kGateUp) ? BN / 2 : BN;   // output columns per tile
    const int n_tiles_n = g.n_out / NCOL;
    int tile, nt;
    prefill_tile_of_block(n_tiles_n, g.group_m, tile, nt);
    if (tile >= g.meta[kMetaTiles]) return;
    const int2 ti = g.tiles[tile];                     // (expert, tile of the expert)
    const int e = ti.x, n_e = g.exp_cnt[e];
    const int first = expert_tile_first(n_e, ti.y, BM);
    const int rows = expert_tile_first(n_e, ti.y + 1, BM) - first;
    const int row0 = g.exp_off[e] + first;
    const int c0 = nt * NCOL;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const int64_t krow = static_cast<int64_t>(g.kd) * EB;     // bytes per weight row

    // MFMA row tiles of this wave that hold rows of the expert (wave-uniform; a prefix of
    // the wave's tiles): the others skip their loads, LDS reads and MFMAs.
    const int ntiles = (rows + 31) / 32;
    const int mvalid = __builtin_amdgcn_readfirstlane(min(MI, max(0, (ntiles - wm + 1) / 2)));

    // Direct-to-LDS assignment.  A: wave (wm, wn) moves rows (wm + 2 i) * 32 + 16 wn +
    // lane/4 of each of its live row tiles i (the rows the pair (wm, 0), (wm, 1) reads);
    // rows past the expert's end inside a live tile re-load its last row (never read
    // back).  B: wave w moves rows w*64 + 16 j + lane/4 (j < 4).  Lane i fetches the
    // global chunk that belongs in LDS slot i % 4.
    const int dr = lane >> 2, soff = dma_chunk_offset(lane);
    const uint8_t* ag[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int rr = min((wm + 2 * i) * 32 + 16 * wn + dr, rows - 1);
        const int64_t arow = GATHER ? g.pair_of_row[row0 + rr] / g.topk : static_cast<int64_t>(row0 + rr);
        ag[i] = static_cast<const uint8_t*>(g.a) + arow * g.lda * EB + soff;
    }
    // B rows of wave w are affine in j (for gate/up, waves 0-1 move gate rows, 2-3 up rows)
    const uint8_t* bg;
    {
        const int r = wave * 64 + dr;
        int64_t wrow;
        if (MODE == kGateUp) wrow = (wave < 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        else wrow = c0 + r;
        bg = static_cast<const uint8_t*>(g.w) + (static_cast<int64_t>(e) * nw + wrow) * krow + soff;
    }
    const int64_t bstep = 16 * krow;      // bytes between B rows j and j + 1

    // FP8 weight-scale exponents: lane l holds the E8M0 code of K block l (gate-column
    // block in s_lo, up-column block in s_hi for gate/up; this wave's column block for
    // down).  kd / 128 <= 64 K blocks (hidden and inter are at most 8192).
    int s_lo = kUnitScale, s_hi = kUnitScale;
    if constexpr (FP8) {
        const int kb_n = g.kd / 128;
        const float* r_lo;
        const float* r_hi;
        const float* wsc = static_cast<const float*>(g.w_scale);
        if (MODE == kGateUp) {
            r_lo = wsc + (static_cast<int64_t>(e) * (nw / 128) + c0 / 128) * kb_n;
            r_hi = wsc + (static_cast<int64_t>(e) * (nw / 128) + (g.n_out + c0) / 128) * kb_n;
        } else {
            r_lo = wsc + (static_cast<int64_t>(e) * (nw / 128) + (c0 + wn * 128) / 128) * kb_n;
            r_hi = r_lo;
        }
        const int l = min(lane, kb_n - 1);
        s_lo = (__float_as_uint(r_lo[l]) >> 23) & 0xff;
        s_hi = (__float_as_uint(r_hi[l]) >> 23) & 0xff;
    }

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
    for (int i = 0; i < MI; ++i) arow_l[i] = (wm + 2 * i) * 32 + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        brow_l[i] = (MODE == kGateUp) ? ((i < 2) ? wn * 64 + i * 32 : BN / 2 + wn * 64 + (i - 2) * 32) + l32
                                      : wn * 128 + i * 32 + l32;
    }
    const int nk = g.kd / BK;          // even: hidden and inter are multiples of 2 * BK

    // The K loop is instantiated per count MV of live row tiles, so no instance tests them.
    auto k_loop = [&](auto mv_tag) {
        constexpr int MV = decltype(mv_tag)::value;
        constexpr int PER = MV + 4;                     // direct-to-LDS loads per stage and wave
        constexpr int NM = (FP8 ? 4 : 8) * MV;          // MFMAs per stage
        constexpr int NR = MV > 0 ? 2 * (MV + 4) : 0;   // 16-byte LDS reads per stage
        auto dma = [&](int slot, int kt) {
            uint8_t* As = smem + slot * kStageBytes;
            uint8_t* Bs = As + BM * kStageRowBytes;
            const int64_t kb = static_cast<int64_t>(kt) * kStageRowBytes;
#pragma unroll
            for (int i = 0; i < MI; ++i)
                if (i < MV) lds_dma16(ag[i] + kb, As + ((wm + 2 * i) * 32 + 16 * wn) * kStageRowBytes);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lds_dma16(bg + j * bstep + kb, Bs + (wave * 64 + j * 16) * kStageRowBytes);
        };
        auto rd = [&](const uint8_t* T, int row, int c) {
            return *reinterpret_cast<const u32x4*>(T + stage_offset(row, c));
        };
        auto load_frags = [&](StageFrags<FP8>& f, int slot) {
            const uint8_t* As = smem + slot * kStageBytes;
            const uint8_t* Bs = As + BM * kStageRowBytes;
            if constexpr (FP8) {
                // 32 bytes per lane: K values 32 lh .. 32 lh + 31 = chunks 2 lh, 2 lh + 1
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) f.a[mi] = join8(rd(As, arow_l[mi], 2 * lh), rd(As, arow_l[mi], 2 * lh + 1));
                if (MV > 0) {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        f.b[ni] = join8(rd(Bs, brow_l[ni], 2 * lh), rd(Bs, brow_l[ni], 2 * lh + 1));
                }
            } else {
                // K step ks: 16 bytes per lane, chunk 2 ks + lh
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        if (mi < MV) f.a[ks][mi] = __builtin_bit_cast(bf16x8, rd(As, arow_l[mi], 2 * ks + lh));
                    if (MV > 0) {
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            f.b[ks][ni] = __builtin_bit_cast(bf16x8, rd(Bs, brow_l[ni], 2 * ks + lh));
                    }
                }
            }
        };
        auto mfma_stage = [&](const StageFrags<FP8>& f, int kt) {
            if constexpr (FP8) {
                const int kb = kt >> 1;                 // 128-wide K block of this stage
                const int sc_lo = __builtin_amdgcn_readlane(s_lo, kb);
                const int sc_hi = __builtin_amdgcn_readlane(s_hi, kb);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) {
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) {
                            const int sb = (MODE == kGateUp && ni >= 2) ? sc_hi : sc_lo;
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0, kUnitScale, 0, sb);
                        }
                    }
            } else {
                (void)kt;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        if (mi < MV) {
#pragma unroll
                            for (int ni = 0; ni < 4; ++ni)
                                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks][mi], f.b[ks][ni],
                                                                                      acc[mi][ni], 0, 0, 0);
                        }
            }
        };

        StageFrags<FP8> f0, f1;
#pragma unroll
        for (int s = 0; s < NST; ++s) dma(s, min(s, nk - 1));
        wait_lds_dma<(NST - 1) * PER>();
        lds_pipeline_barrier();
        load_frags(f0, 0);
        // One iteration: wait for stage j + 1, then MFMAs of stage j (registers) with the
        // LDS reads of stage j + 1 and the loads of stage j + NST (into slot j % NST)
        // between them.  Unrolled by two so the fragment buffers alternate statically; the
        // body is branch-free: past the end the slab index is clamped and the last
        // iterations re-load the last slab into slots nothing reads any more.
        auto iteration = [&](StageFrags<FP8>& cur, StageFrags<FP8>& nxt, int j, int slot) {
            const int nslot = (slot + 1 == NST) ? 0 : slot + 1;
            __builtin_amdgcn_sched_barrier(0);
            wait_lds_dma<(NST - 2) * PER>();
            lds_pipeline_barrier();
            __builtin_amdgcn_sched_barrier(0);
            mfma_stage(cur, j);
            load_frags(nxt, nslot);
            dma(slot, min(j + NST, nk - 1));
            sched_interleave<NM, NR, PER>();
            __builtin_amdgcn_sched_barrier(0);
            return nslot;
        };
        int slot = 0;
        for (int j = 0; j < nk; j += 2) {
            slot = iteration(f0, f1, j, slot);
            slot = iteration(f1, f0, j + 1, slot);
        }
    };
    dispatch_row_tiles<MI>(mvalid, k_loop);

    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = (wm + 2 * mi) * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            if (m >= rows) continue;
            float sa = 1.0f;
            if constexpr (FP8) {
                const int64_t ar = GATHER ? g.pair_of_row[row0 + m] / g.topk : static_cast<int64_t>(row0 + m);
                sa = g.a_scale[ar];
            }
            uint16_t* orow = out + static_cast<int64_t>(row0 + m) * g.ldo;
            if (MODE == kGateUp) {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    orow[c0 + wn * 64 + ni * 32 + l32] =
                        f32_to_bf16_bits(silu(acc[mi][ni][i] * sa) * (acc[mi][ni + 2][i] * sa));
            } else {
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    orow[c0 + wn * 128 + ni * 32 + l32] = f32_to_bf16_bits(acc[mi][ni][i] * sa);
            }
        }
    }
}

template <int MODE, bool GATHER, bool FP8>
static void launch_prefill_inst(hipStream_t st, const GroupedGemmArgs& g, int blocks) {
    static bool attr_set = false;     // the LDS opt-in is per kernel, set on first use
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_prefill<MODE, GATHER, FP8>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
        attr_set = true;
    }
    gemm_prefill<MODE, GATHER, FP8><<<blocks, 256, kLdsBytes, st>>>(g);
}

template <bool FP8>
static void launch_prefill_dtype(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, int blocks) {
    if (mode == kGateUp) {
        if (g.gather) launch_prefill_inst<kGateUp, true, FP8>(st, g, blocks);
        else launch_prefill_inst<kGateUp, false, FP8>(st, g, blocks);
    } else {
        if (g.gather) launch_prefill_inst<kDown, true, FP8>(st, g, blocks);
        else launch_prefill_inst<kDown, false, FP8>(st, g, blocks);
    }
}

void launch_gemm_prefill(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, bool fp8) {
    if (g.max_tiles == 0) return;
    const int ncol = (mode == kGateUp) ? 128 : 256;
    // every (row tile, column tile) of whole groups of group_m row tiles, in whole XCD chunks
    const int64_t groups = (g.max_tiles + g.group_m - 1) / g.group_m;
    const int blocks = static_cast<int>((groups * g.group_m * (g.n_out / ncol) + 255) / 256 * 256);
    if (fp8) launch_prefill_dtype<true>(st, mode, g, blocks);
    else launch_prefill_dtype<false>(st, mode, g, blocks);
}

}  // namespace beam
