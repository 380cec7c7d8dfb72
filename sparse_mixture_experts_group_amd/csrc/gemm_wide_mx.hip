// Grouped expert GEMMs for many rows per expert with MXFP4 weights (OCP MX: FP4 E2M1
// elements, one E8M0 scale per 32 along K) and E4M3 activations (one FP32 scale per
// row): the LDS-tiled MFMA GEMM with K stages of 128 values.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
// Tiles, wave roles and block order are those of gemm_prefill.hip; the MFMA is
// v_mfma_scale_f32_32x32x64_f8f6f4 computing the transposed tile (the epilogue of
// tile_epilogue.cuh) with the FP4 weights as its A operand: a lane holds one 32-value MX
// block of its weight row and takes that block's E8M0 byte as its scale (the FP4 lane
// layout measured on gfx950, the same for either operand; the E4M3 activation lane that
// pairs with it holds K 16 h .. 16 h + 15 and 32 + 16 h .. 32 + 16 h + 15 of the 64-wide
// step, h the lane's half).
//
// Why 128-value stages: the 64-value stages of gemm_prefill.hip fetch FP4 weight rows in
// 32-byte pieces, a quarter of an L2 line per request; here a stage holds 128 bytes of
// every activation row and 64 bytes of every weight row (32 KB + 16 KB).  Two activation
// and three weight slots (112 KB) leave 48 KB of LDS for the tile's block scales, so a
// K slice is at most 6144 long (the launcher splits longer reductions or falls back).
#include "common.cuh"
#include "kernels.h"
#include "tile_epilogue.cuh"

namespace beam {

namespace {
constexpr int kUnitScale = 0x7f;                 // E8M0 code of 2^0
constexpr int kMxARowBytes = 128;                // activation bytes per row and stage (128 E4M3)
constexpr int kMxBRowBytes = 64;                 // weight bytes per row and stage (128 FP4)
constexpr int kMxASlotBytes = 256 * kMxARowBytes;
constexpr int kMxBSlotBytes = 256 * kMxBRowBytes;
constexpr int kMxASlots = 2, kMxBSlots = 3;
constexpr int kMxStageLds = kMxASlots * kMxASlotBytes + kMxBSlots * kMxBSlotBytes;
constexpr int kMxMaxKlen = (160 * 1024 - kMxStageLds) / 256 * 32;   // scales: 256 rows x klen/32
static_assert(kMxMaxKlen >= 6144, "LDS budget");

// Activation rows (128 bytes): chunk c of row r in slot c ^ ((r >> 1) & 7); a DMA
// instruction covers 8 rows, lane i landing in row base + i / 8, slot i % 8.
__device__ __forceinline__ int mx_a_offset(int row, int chunk) {
    return row * kMxARowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}
__device__ __forceinline__ int mx_a_dma_chunk(int lane, int odd) {   // odd: bit 3 of the base row
    return ((lane & 7) ^ (((lane >> 4) + 4 * odd) & 7)) << 4;
}
// Weight rows (64 bytes): chunk c of row r in slot c ^ ((r >> 2) & 3); a DMA instruction
// covers 16 rows (base a multiple of 16), lane i landing in row base + i / 4, slot i % 4.
__device__ __forceinline__ int mx_b_offset(int row, int chunk) {
    return row * kMxBRowBytes + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
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

// Fragments of one 64-wide K step for one wave.
struct MxFrags { i32x8 a[4]; u32x4 b[4]; };
}  // namespace

// Pipeline per stage kt (2 K steps of 64): K step 0 runs its MFMAs while reading step 1's
// fragments; before step 1 every wave waits until stage kt + 1 has landed (only the weight
// loads of stage kt + 2 may still be in flight) and meets the others, then loads the
// activations of stage kt + 2 and the weights of stage kt + 3 into the slots stage kt
// drained, runs step 1's MFMAs and reads stage kt + 1's first fragments.
//
// SPLIT: as in gemm_prefill.hip, the GEMMs of a single weight set split K into
// g.k_slices slices (FP32 partial sums) over a flat block order.
template <int MODE, bool GATHER, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_wide_mx(GroupedGemmArgs g) {
    constexpr int BM = kPrefillBM, BN = 256, MI = 4, NI = 4;
    constexpr int BK = 128;                             // K per stage
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NCOL = (MODE == kGateUp) ? BN / 2 : BN;   // output columns per tile
    const int n_tiles_n = g.n_out / NCOL;
    int tile, nt, kz = 0;
    if constexpr (SPLIT) {
        const int lin = blockIdx.x;
        kz = lin % g.k_slices;
        const int rest = lin / g.k_slices;
        nt = rest % n_tiles_n;
        tile = rest / n_tiles_n;
    } else {
        prefill_tile_of_block(n_tiles_n, g.group_m, tile, nt);
    }
    if (tile >= g.meta[kMetaTiles]) return;
    const int2 ti = g.tiles[tile];                     // (expert, tile of the expert)
    const int e = ti.x, n_e = g.exp_cnt[e];
    const int first = expert_tile_first(n_e, ti.y, BM);
    const int rows = expert_tile_first(n_e, ti.y + 1, BM) - first;
    const int row0 = g.exp_off[e] + first;
    const int c0 = nt * NCOL;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    const int64_t krow = g.kd / 2;                               // weight bytes per row
    const int klen = SPLIT ? g.kd / g.k_slices : g.kd;           // K slice of this block
    const int kbeg = SPLIT ? kz * klen : 0;

    const int ntiles = (rows + 31) / 32;
    const int mvalid = __builtin_amdgcn_readfirstlane(min(MI, max(0, (ntiles - wm + 1) / 2)));

    // Direct-to-LDS assignment.  Activations: 8 rows x 128 bytes per instruction, wave
    // (wm, wn) moving rows (wm + 2 i) * 32 + 16 wn + 8 h + lane / 8 (h < 2) of its live row
    // tiles (rows past the expert's end re-load its last row).  Weights: 16 rows x 64 bytes
    // per instruction, wave w moving rows w * 64 + 16 j + lane / 4 (j < 4; for gate/up
    // waves 0-1 move gate rows, 2-3 up rows).  Block-uniform bases + 32-bit lane offsets
    // (the launcher checks the activation extent; one expert's weights always fit).
    const uint8_t* abase = static_cast<const uint8_t*>(g.a) + kbeg;
    uint32_t aoff[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rr = min((wm + 2 * i) * 32 + 16 * wn + 8 * h + (lane >> 3), rows - 1);
            const int64_t arow = GATHER ? g.pair_of_row[row0 + rr] / g.topk : static_cast<int64_t>(row0 + rr);
            aoff[i][h] = static_cast<uint32_t>(arow * g.lda) + mx_a_dma_chunk(lane, h);
        }
    auto weight_row = [&](int r) -> int {                // block row r (0..255) -> weight row
        if (MODE == kGateUp) return (r < BN / 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        return c0 + r;
    };
    const uint8_t* bbase = static_cast<const uint8_t*>(g.w) + static_cast<int64_t>(e) * nw * krow + kbeg / 2;
    const uint32_t boff = static_cast<uint32_t>(weight_row(wave * 64 + (lane >> 2)) * krow) + dma_chunk_offset(lane);
    const uint32_t bstep = static_cast<uint32_t>(16 * krow);   // bytes between B rows j and j + 1
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(abase, g.a_rows * g.lda - kbeg);
    const __amdgpu_buffer_rsrc_t rsrc_b = buffer_rsrc(bbase, nw * krow - kbeg / 2);

    // The tile's E8M0 block scales of its K slice: 256 weight rows x klen / 32 codes after
    // the operand slots (thread t copies row t).
    const int srow = klen / 32;
    uint8_t* ssc = smem + kMxStageLds;
    {
        const uint8_t* src = static_cast<const uint8_t*>(g.w_scale) +
                             (static_cast<int64_t>(e) * nw + weight_row(tid)) * (g.kd / 32) + kbeg / 32;
        for (int c = 0; c < srow; c += 16)
            *reinterpret_cast<u32x4*>(ssc + tid * srow + c) = *reinterpret_cast<const u32x4*>(src + c);
        // complete before the pipeline: its waits count the direct-to-LDS loads alone
        __syncthreads();
    }

    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

    const int l32 = lane & 31, lh = lane >> 5;
    int arow_l[MI], brow_l[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) arow_l[i] = (wm + 2 * i) * 32 + l32;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        brow_l[i] = (MODE == kGateUp) ? ((i < 2) ? wn * 64 + i * 32 : BN / 2 + wn * 64 + (i - 2) * 32) + l32
                                      : wn * 128 + i * 32 + l32;
    }
    const int nk = klen / BK;          // slices are multiples of 512

    auto k_loop = [&](auto mv_tag) {
        constexpr int MV = decltype(mv_tag)::value;
        constexpr int NM = MV * NI;                      // MFMAs per K step
        constexpr int NR = MV == 0 ? 0 : 2 * MV + NI;    // LDS reads per K step
        auto dma_a = [&](int slot, int kt) {            // activations of stage kt
            uint8_t* As = smem + slot * kMxASlotBytes;
            const int ks = kt * kMxARowBytes;
#pragma unroll
            for (int i = 0; i < MI; ++i)
                if (i < MV) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        lds_dma16_buf(rsrc_a, As + ((wm + 2 * i) * 32 + 16 * wn + 8 * h) * kMxARowBytes, aoff[i][h], ks);
                }
        };
        auto dma_b = [&](int slot, int kt) {            // weights of stage kt (4 loads)
            uint8_t* Bs = smem + kMxASlots * kMxASlotBytes + slot * kMxBSlotBytes;
            const int ks = kt * kMxBRowBytes;
#pragma unroll
            for (int j = 0; j < 4; ++j) lds_dma16_buf(rsrc_b, Bs + (wave * 64 + 16 * j) * kMxBRowBytes, boff + j * bstep, ks);
        };
        // fragments of K step s (64 values) of a stage whose operands sit in aslot, bslot
        auto load_frags = [&](MxFrags& f, int aslot, int bslot, int s) {
            const uint8_t* As = smem + aslot * kMxASlotBytes;
            const uint8_t* Bs = smem + kMxASlots * kMxASlotBytes + bslot * kMxBSlotBytes;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                if (mi < MV)
                    f.a[mi] = join8(*reinterpret_cast<const u32x4*>(As + mx_a_offset(arow_l[mi], 4 * s + lh)),
                                    *reinterpret_cast<const u32x4*>(As + mx_a_offset(arow_l[mi], 4 * s + 2 + lh)));
            if (MV > 0) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    f.b[ni] = *reinterpret_cast<const u32x4*>(Bs + mx_b_offset(brow_l[ni], 2 * s + lh));
            }
        };
        auto mfma_step = [&](const MxFrags& f, int kt, int s) {
            if (MV > 0) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    // E8M0 code of this lane's column, MX block 4 kt + 2 s + lh of the slice
                    const int sb = ssc[brow_l[ni] * srow + 4 * kt + 2 * s + lh];
                    const i32x8 bb = fp4_operand(f.b[ni]);
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        if (mi < MV)
                            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                bb, f.a[mi], acc[mi][ni], 4, 0, 0, sb, 0, kUnitScale);
                }
            }
        };

        MxFrags f0, f1;
        // The loop body is branch-free (a branch would split the fragment registers into
        // copies at its join): stage indices past the end are clamped, and the last
        // iterations re-load the last stage into slots nothing reads any more, so every
        // stage issues the same loads and every wait count is fixed.
        // Prologue order: A0 B0 A1 B1; wait for stage 0 (A0, B0).  Issue order in the
        // loop: B(kt + 2) during K step 0 of stage kt, A(kt + 2) during step 1.
        dma_a(0, 0);
        dma_b(0, 0);
        dma_a(1, min(1, nk - 1));
        dma_b(1, min(1, nk - 1));
        wait_lds_dma<2 * MV + 4>();
        lds_pipeline_barrier();
        load_frags(f0, 0, 0, 0);
        int bslot = 0;                                   // weight slot of stage kt (kt % 3)
        for (int kt = 0; kt < nk; ++kt) {
            const int aslot = kt & 1;
            const int bnext = (bslot == kMxBSlots - 1) ? 0 : bslot + 1;
            const int bfree = (bslot == 0) ? kMxBSlots - 1 : bslot - 1;      // stage kt - 1's slot
            // step 0: the next step's fragments, then the weights of stage kt + 2
            __builtin_amdgcn_sched_barrier(0);
            mfma_step(f0, kt, 0);
            load_frags(f1, aslot, bslot, 1);
            dma_b(bfree, min(kt + 2, nk - 1));
            if constexpr (MV > 0) __builtin_amdgcn_sched_group_barrier(0x100, NI, 0);   // the step's scale reads
            sched_reads_then_loads<NM, NR, 4>();
            __builtin_amdgcn_sched_barrier(0);
            // step 1.  Issue order so far ends ... A(kt+1), B(kt+2): stage kt + 1 has landed
            // once at most the 4 weight loads of stage kt + 2 are in flight.
            wait_lds_dma<4>();
            lds_pipeline_barrier();
            __builtin_amdgcn_sched_barrier(0);
            mfma_step(f1, kt, 1);
            load_frags(f0, aslot ^ 1, bnext, 0);
            dma_a(aslot, min(kt + 2, nk - 1));           // into the slot stage kt drained
            if constexpr (MV > 0) __builtin_amdgcn_sched_group_barrier(0x100, NI, 0);   // the step's scale reads
            sched_reads_then_loads<NM, NR, 2 * MV>();
            __builtin_amdgcn_sched_barrier(0);
            bslot = bnext;
        }
        wait_lds_dma<0>();      // the tail's re-loads land before the block's LDS is released
    };
    dispatch_row_tiles<MI>(mvalid, k_loop);

    // down: 256-byte row segments per wave, staged through LDS for whole-row stores;
    // gate/up (128-byte segments) and FP32 partial sums: stored from the registers
    if constexpr (SPLIT || MODE == kGateUp) {
        store_wide_tile<MODE, GATHER, true, SPLIT, 2>(g, acc, rows, row0, c0, wm, wn, lane, kz);
    } else {
        __syncthreads();                 // every wave is out of its K loop: the LDS is free
        store_wide_tile_bf16<MODE, GATHER, true, 2>(g, acc, rows, row0, c0, wm, wn, wave, lane, smem);
    }
}

template <int MODE, bool GATHER, bool SPLIT>
static void launch_wide_mx_inst(hipStream_t st, const GroupedGemmArgs& g, int blocks, int ks) {
    lds_opt_in(reinterpret_cast<const void*>(&gemm_wide_mx<MODE, GATHER, SPLIT>), 160 * 1024);
    // the pipeline's slots and scales, or the BF16 epilogue's staging if larger
    size_t lds = kMxStageLds + 256 * static_cast<size_t>(g.kd / ks / 32);
    if (!SPLIT && MODE == kDown && lds < wide_epilogue_lds(MODE)) lds = wide_epilogue_lds(MODE);
    if (SPLIT) {
        GroupedGemmArgs gs = g;
        gs.k_slices = ks;
        gemm_wide_mx<MODE, GATHER, SPLIT><<<blocks, 256, lds, st>>>(gs);
    } else {
        gemm_wide_mx<MODE, GATHER, SPLIT><<<blocks, 256, lds, st>>>(g);
    }
}

bool wide_mx_supported(const GroupedGemmArgs& g, int ks) {
    const int klen = g.kd / ks;
    return klen <= kMxMaxKlen && klen % 512 == 0;
}

int launch_gemm_wide_mx(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, int ks) {
    if (g.max_tiles == 0) return 1;
    const int ncol = (mode == kGateUp) ? 128 : 256;
    if (ks > 1) {
        // split K only for a single weight set (rows in token order, no gather); the grid
        // enumerates every (row tile bound, column tile, slice)
        const int nb = g.max_tiles * (g.n_out / ncol) * ks;
        if (mode == kGateUp) launch_wide_mx_inst<kGateUp, false, true>(st, g, nb, ks);
        else launch_wide_mx_inst<kDown, false, true>(st, g, nb, ks);
        return ks;
    }
    // every (row tile, column tile) of whole groups of group_m row tiles, in whole XCD chunks
    const int64_t groups = (g.max_tiles + g.group_m - 1) / g.group_m;
    const int blocks = static_cast<int>((groups * g.group_m * (g.n_out / ncol) + 255) / 256 * 256);
    if (mode == kGateUp) {
        if (g.gather) launch_wide_mx_inst<kGateUp, true, false>(st, g, blocks, 1);
        else launch_wide_mx_inst<kGateUp, false, false>(st, g, blocks, 1);
    } else {
        if (g.gather) launch_wide_mx_inst<kDown, true, false>(st, g, blocks, 1);
        else launch_wide_mx_inst<kDown, false, false>(st, g, blocks, 1);
    }
    return 1;
}

}  // namespace beam
