// Grouped expert GEMMs for many rows per expert (prefill-sized batches) on the gfx950
// matrix cores, FP32 accumulation; BF16, FP8 (OCP E4M3FN) or MXFP4 (OCP MX: FP4 E2M1
// elements with an E8M0 scale per 32 along K) weights.
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
// FP8: weights carry one FP32 scale per 128 x 128 block, whose exponent the f8f6f4 MFMA
// applies itself as the E8M0 scale of its B operand (the FP32 scale's exponent field is
// the E8M0 code).  Power-of-two scales need nothing more; otherwise (MANT) the
// significand m in [1, 2) of each block scale is folded by keeping the accumulators in
// units of the current block's m: before the MFMAs of K block kb they are multiplied by
// m[kb-1] / m[kb], after the last block by m[last].  MXFP4: the FP4 B
// operand of a lane holds one 32-value MX block of its column, whose E8M0 scale is the
// lane's B scale byte; the block's scales are staged in LDS once.  Activations (FP8 and
// MXFP4 weights) are E4M3 with one FP32 scale per row, applied in the epilogue.
#include "common.cuh"
#include "kernels.h"

namespace beam {

namespace {
constexpr int kUnitScale = 0x7f;                // E8M0 code of 2^0
enum : int { kWtBf16 = 0, kWtFp8 = 1, kWtMxfp4 = 2 };

// K advances per LDS stage: A rows hold 64 bytes (32 BF16 or 64 E4M3
// values), B rows 64 bytes (BF16, FP8) or 32 bytes (64 packed FP4 values).
template <int WT> constexpr int b_row_bytes() { return WT == kWtMxfp4 ? 32 : kStageRowBytes; }
template <int WT> constexpr int stage_bytes() { return kPrefillBM * kStageRowBytes + 256 * b_row_bytes<WT>(); }
constexpr int kStages = 4;
constexpr int kMxfp4MaxKd = 8192;               // LDS holds the block's 256 x kd/32 scales
constexpr int kFp8MaxKb = kFp8PrefillMaxKd / 128;   // FP8: K blocks of a reduction
// LDS after the stages: MXFP4 block scales (256 rows x kd/32 codes), or for FP8 with more
// than 64 K blocks two rows of kd/128 block-scale codes (16-byte aligned size) followed
// by two rows of kd/128 FP32 significand ratios
constexpr int fp8_code_bytes(int kb_n) { return (2 * kb_n + 15) / 16 * 16; }
template <int WT> constexpr size_t lds_bytes_max() {
    return kStages * stage_bytes<WT>() +
           (WT == kWtMxfp4 ? 256 * (kMxfp4MaxKd / 32)
                           : (WT == kWtFp8 ? fp8_code_bytes(kFp8MaxKb) + 2 * sizeof(float) * kFp8MaxKb : 0));
}
static_assert(lds_bytes_max<kWtFp8>() <= 160 * 1024 && lds_bytes_max<kWtMxfp4>() <= 160 * 1024, "LDS budget");

// FP4 rows of 32 bytes: chunk c of row r in slot c ^ ((r >> 3) & 1), so the 16 rows one
// fragment read serves per LDS cycle cover all banks.
__device__ __forceinline__ int fp4_offset(int row, int chunk) {
    return row * 32 + ((chunk ^ ((row >> 3) & 1)) << 4);
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

// Fragments of one LDS stage for one wave: BF16 - two 16-wide K steps of 8 values per
// lane; FP8 - one 64-wide K step of 32 values per lane; MXFP4 - A as FP8, B 32 FP4
// values (16 bytes) per lane.
template <int WT> struct StageFrags;
template <> struct StageFrags<kWtBf16> { bf16x8 a[2][4]; bf16x8 b[2][4]; };
template <> struct StageFrags<kWtFp8> { i32x8 a[4]; i32x8 b[4]; };
template <> struct StageFrags<kWtMxfp4> { i32x8 a[4]; u32x4 b[4]; };
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
//
// SPLIT: the GEMMs of a single weight set, which alone have too few tiles for the chip,
// split K into g.k_slices slices and write FP32 partial sums.  The 1-D grid enumerates
// (row tile, column tile, slice) with the slice fastest and no XCD grouping, so
// consecutive blocks -- which the dispatcher deals out over the XCDs in turn -- spread
// the few tiles over the whole chip.
template <int MODE, bool GATHER, int WT, bool MANT, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_prefill(GroupedGemmArgs g) {
    static_assert(WT == kWtFp8 || !MANT, "block-scale significands are an FP8 feature");
    constexpr int BM = kPrefillBM, BN = 256, MI = 4, NST = kStages;
    constexpr bool Q8 = WT != kWtBf16;                  // E4M3 activations with row scales
    constexpr int EB = Q8 ? 1 : 2;                      // bytes per activation element
    constexpr int BK = kStageRowBytes / EB;             // K per stage
    constexpr int BRB = b_row_bytes<WT>();              // bytes per B row per stage
    constexpr int SB = stage_bytes<WT>();
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
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nw = (MODE == kGateUp) ? 2 * static_cast<int64_t>(g.n_out) : g.n_out;
    // bytes per weight row (MXFP4: two values per byte)
    const int64_t krow = (WT == kWtMxfp4) ? g.kd / 2 : static_cast<int64_t>(g.kd) * EB;
    // K slice of this block
    const int klen = SPLIT ? g.kd / g.k_slices : g.kd;
    const int kbeg = SPLIT ? kz * klen : 0;
    const int64_t kbeg_w = (WT == kWtMxfp4) ? kbeg / 2 : static_cast<int64_t>(kbeg) * EB;   // weight bytes

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
        ag[i] = static_cast<const uint8_t*>(g.a) + (arow * g.lda + kbeg) * EB + soff;
    }
    // B rows of wave w are affine in j (for gate/up, waves 0-1 move gate rows, 2-3 up rows).
    // BF16 / FP8: rows w*64 + 16 j + lane/4, lane i fetching the chunk of LDS slot i % 4;
    // MXFP4 (32-byte rows): rows w*64 + 32 j + lane/2, chunk of slot i % 2.
    constexpr int BRPI = (WT == kWtMxfp4) ? 32 : 16;     // B rows per DMA instruction
    constexpr int BJ = 64 / BRPI;                         // B DMA instructions per wave
    const int bdr = (WT == kWtMxfp4) ? (lane >> 1) : dr;
    const int bsoff = (WT == kWtMxfp4) ? (((lane & 1) ^ ((lane >> 4) & 1)) << 4) : soff;
    auto weight_row = [&](int r) -> int64_t {            // block row r (0..255) -> weight row
        if (MODE == kGateUp) return (r < BN / 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        return c0 + r;
    };
    const uint8_t* bg = static_cast<const uint8_t*>(g.w) +
                        (static_cast<int64_t>(e) * nw + weight_row(wave * 64 + bdr)) * krow + kbeg_w + bsoff;
    const int64_t bstep = BRPI * krow;    // bytes between B rows j and j + 1

    // FP8 weight-scale exponents: lane l holds the E8M0 code of K block l (gate-column
    // block in s_lo, up-column block in s_hi for gate/up; this wave's column block for
    // down), and for MANT the significand ratio m[l-1] / m[l] (q_lo, q_hi; 1 for l = 0);
    // m_end_* is the last block's significand.  Blocks from 64 on are read from LDS (see
    // below).
    int s_lo = kUnitScale, s_hi = kUnitScale;
    float q_lo = 1.0f, q_hi = 1.0f, m_end_lo = 1.0f, m_end_hi = 1.0f;
    uint8_t* fsc = smem + NST * SB;          // FP8, kd / 128 > 64: [2][kd / 128] codes
    float* fsq = reinterpret_cast<float*>(fsc + fp8_code_bytes(klen / 128));   // then [2][kd / 128] ratios
    if constexpr (WT == kWtFp8) {
        const int kb_all = g.kd / 128, kb_n = klen / 128;     // K blocks of the row, of the slice
        const float* r_lo;
        const float* r_hi;
        const float* wsc = static_cast<const float*>(g.w_scale) + kbeg / 128;
        if (MODE == kGateUp) {
            r_lo = wsc + (static_cast<int64_t>(e) * (nw / 128) + c0 / 128) * kb_all;
            r_hi = wsc + (static_cast<int64_t>(e) * (nw / 128) + (g.n_out + c0) / 128) * kb_all;
        } else {
            r_lo = wsc + (static_cast<int64_t>(e) * (nw / 128) + (c0 + wn * 128) / 128) * kb_all;
            r_hi = r_lo;
        }
        const int l = min(lane, kb_n - 1);
        s_lo = scale_e8m0(r_lo[l]);
        s_hi = scale_e8m0(r_hi[l]);
        if constexpr (MANT) {
            const int lp = max(l - 1, 0);
            q_lo = __fdiv_rn(scale_mantissa(r_lo[lp]), scale_mantissa(r_lo[l]));
            q_hi = __fdiv_rn(scale_mantissa(r_hi[lp]), scale_mantissa(r_hi[l]));
            m_end_lo = scale_mantissa(r_lo[kb_n - 1]);
            m_end_hi = scale_mantissa(r_hi[kb_n - 1]);
        }
        if (kb_n > 64) {
            // the codes (and ratios) of every K block in LDS: row 0 the gate (down: wn = 0)
            // column block, row 1 the up (down: wn = 1) block; waves 0 and 1 write them
            if (wave < 2) {
                // (for down, r_lo is this wave's own column block: wn = wave)
                const float* src = (MODE == kGateUp) ? (wave == 0 ? r_lo : r_hi) : r_lo;
                for (int i = lane; i < kb_n; i += 64) {
                    fsc[wave * kb_n + i] = static_cast<uint8_t>(scale_e8m0(src[i]));
                    if constexpr (MANT)
                        fsq[wave * kb_n + i] = __fdiv_rn(scale_mantissa(src[max(i - 1, 0)]), scale_mantissa(src[i]));
                }
            }
            // complete before the pipeline: its waits count the direct-to-LDS loads alone
            __syncthreads();
        }
    }
    // MXFP4 block scales: the block's 256 weight rows x klen/32 E8M0 codes of its K slice,
    // staged in LDS after the stages (thread t copies row t; the rows of one half are
    // contiguous).
    const int srow = klen / 32;
    uint8_t* ssc = smem + NST * SB;
    if constexpr (WT == kWtMxfp4) {
        const uint8_t* src = static_cast<const uint8_t*>(g.w_scale) +
                             (static_cast<int64_t>(e) * nw + weight_row(tid)) * (g.kd / 32) + kbeg / 32;
        for (int c = 0; c < srow; c += 16)
            *reinterpret_cast<u32x4*>(ssc + tid * srow + c) = *reinterpret_cast<const u32x4*>(src + c);
        // complete before the pipeline: its waits count the direct-to-LDS loads alone
        __syncthreads();
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
    const int nk = klen / BK;          // even: slices are multiples of 2 * BK

    // The K loop is instantiated per count MV of live row tiles, so no instance tests them.
    auto k_loop = [&](auto mv_tag) {
        constexpr int MV = decltype(mv_tag)::value;
        constexpr int PER = MV + BJ;                    // direct-to-LDS loads per stage and wave
        constexpr int NM = (WT == kWtBf16 ? 8 : 4) * MV;   // MFMAs per stage
        constexpr int NR = MV == 0 ? 0 : (WT == kWtMxfp4 ? 2 * MV + 8 : 2 * (MV + 4));   // LDS reads
        auto dma = [&](int slot, int kt) {
            uint8_t* As = smem + slot * SB;
            uint8_t* Bs = As + BM * kStageRowBytes;
            const int64_t kb = static_cast<int64_t>(kt) * kStageRowBytes;
#pragma unroll
            for (int i = 0; i < MI; ++i)
                if (i < MV) lds_dma16(ag[i] + kb, As + ((wm + 2 * i) * 32 + 16 * wn) * kStageRowBytes);
            const int64_t kbb = static_cast<int64_t>(kt) * BRB;
#pragma unroll
            for (int j = 0; j < BJ; ++j)
                lds_dma16(bg + j * bstep + kbb, Bs + (wave * 64 + j * BRPI) * BRB);
        };
        auto rd = [&](const uint8_t* T, int row, int c) {
            return *reinterpret_cast<const u32x4*>(T + stage_offset(row, c));
        };
        auto load_frags = [&](StageFrags<WT>& f, int slot) {
            const uint8_t* As = smem + slot * SB;
            const uint8_t* Bs = As + BM * kStageRowBytes;
            if constexpr (WT == kWtFp8) {
                // 32 bytes per lane: K values 32 lh .. 32 lh + 31 = chunks 2 lh, 2 lh + 1
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) f.a[mi] = join8(rd(As, arow_l[mi], 2 * lh), rd(As, arow_l[mi], 2 * lh + 1));
                if (MV > 0) {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        f.b[ni] = join8(rd(Bs, brow_l[ni], 2 * lh), rd(Bs, brow_l[ni], 2 * lh + 1));
                }
            } else if constexpr (WT == kWtMxfp4) {
                // B lane: its column's MX block lh (K 32 lh .. 32 lh + 31, 16 bytes); the E4M3
                // A lane that pairs with it holds K 16 lh .. +15 and 32 + 16 lh .. +15 (the
                // operand layout of this MFMA with an FP4 B, measured on gfx950)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) f.a[mi] = join8(rd(As, arow_l[mi], lh), rd(As, arow_l[mi], lh + 2));
                if (MV > 0) {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        f.b[ni] = *reinterpret_cast<const u32x4*>(Bs + fp4_offset(brow_l[ni], lh));
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
        // even: kt is even, the first stage of a 128-wide K block (stages are 64 wide),
        // where MANT moves the accumulators into the units of the block's significands
        auto mfma_stage = [&](const StageFrags<WT>& f, int kt, auto even_tag) {
            if constexpr (WT == kWtFp8) {
                const int kb = kt >> 1;                 // 128-wide K block of this stage
                int sc_lo, sc_hi;
                float r_lo = 1.0f, r_hi = 1.0f;
                constexpr bool kRescale = MANT && decltype(even_tag)::value;
                if (kb < 64) {
                    sc_lo = __builtin_amdgcn_readlane(s_lo, kb);
                    sc_hi = __builtin_amdgcn_readlane(s_hi, kb);
                    if constexpr (kRescale) {
                        r_lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q_lo), kb));
                        r_hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q_hi), kb));
                    }
                } else {
                    const int kb_n = klen / 128;
                    const int rl = (MODE == kGateUp ? 0 : wn) * kb_n + kb;
                    sc_lo = fsc[rl];
                    sc_hi = (MODE == kGateUp) ? fsc[kb_n + kb] : sc_lo;
                    if constexpr (kRescale) {
                        r_lo = fsq[rl];
                        r_hi = (MODE == kGateUp) ? fsq[kb_n + kb] : r_lo;
                    }
                }
                if constexpr (kRescale) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        if (mi < MV) {
#pragma unroll
                            for (int ni = 0; ni < 4; ++ni) {
                                const float r = (MODE == kGateUp && ni >= 2) ? r_hi : r_lo;
#pragma unroll
                                for (int i = 0; i < 16; ++i) acc[mi][ni][i] *= r;
                            }
                        }
                }
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
            } else if constexpr (WT == kWtMxfp4) {
                (void)even_tag;
                if (MV > 0) {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        // E8M0 code of this lane's column, MX block 2 kt + lh
                        const int sb = ssc[(brow_l[ni]) * srow + 2 * kt + lh];
                        const i32x8 bb = fp4_operand(f.b[ni]);
#pragma unroll
                        for (int mi = 0; mi < MI; ++mi)
                            if (mi < MV)
                                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    f.a[mi], bb, acc[mi][ni], 0, 4, 0, kUnitScale, 0, sb);
                    }
                }
            } else {
                (void)kt;
                (void)even_tag;
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

        StageFrags<WT> f0, f1;
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
        auto iteration = [&](StageFrags<WT>& cur, StageFrags<WT>& nxt, int j, int slot, auto even_tag) {
            const int nslot = (slot + 1 == NST) ? 0 : slot + 1;
            __builtin_amdgcn_sched_barrier(0);
            wait_lds_dma<(NST - 2) * PER>();
            lds_pipeline_barrier();
            __builtin_amdgcn_sched_barrier(0);
            mfma_stage(cur, j, even_tag);
            load_frags(nxt, nslot);
            dma(slot, min(j + NST, nk - 1));
            sched_interleave<NM, NR, PER>();
            __builtin_amdgcn_sched_barrier(0);
            return nslot;
        };
        int slot = 0;
        for (int j = 0; j < nk; j += 2) {
            slot = iteration(f0, f1, j, slot, std::true_type{});
            slot = iteration(f1, f0, j + 1, slot, std::false_type{});
        }
    };
    dispatch_row_tiles<MI>(mvalid, k_loop);
    if constexpr (MANT) {
        // from the units of the last block's significand back to the block scales
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const float m = (MODE == kGateUp && ni >= 2) ? m_end_hi : m_end_lo;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mi][ni][i] *= m;
            }
    }

    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = (wm + 2 * mi) * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            if (m >= rows) continue;
            float sa = 1.0f;
            if constexpr (Q8) {
                const int64_t ar = GATHER ? g.pair_of_row[row0 + m] / g.topk : static_cast<int64_t>(row0 + m);
                sa = g.a_scale[ar];
            }
            uint16_t* orow = out + static_cast<int64_t>(row0 + m) * g.ldo;
            if constexpr (SPLIT) {
                // FP32 partial sums of the slice: gate then up sums for gate/up (the SwiGLU
                // follows the reduction)
                float* prow = g.part + kz * g.part_slice +
                              static_cast<int64_t>(row0 + m) * (MODE == kGateUp ? 2 * g.n_out : g.ldo);
                if (MODE == kGateUp) {
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        prow[c0 + wn * 64 + ni * 32 + l32] = acc[mi][ni][i] * sa;
                        prow[g.n_out + c0 + wn * 64 + ni * 32 + l32] = acc[mi][ni + 2][i] * sa;
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) prow[c0 + wn * 128 + ni * 32 + l32] = acc[mi][ni][i] * sa;
                }
                continue;
            }
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

template <int MODE, bool GATHER, int WT, bool MANT, bool SPLIT>
static void launch_prefill_inst(hipStream_t st, const GroupedGemmArgs& g, int blocks, int ks) {
    lds_opt_in(reinterpret_cast<const void*>(&gemm_prefill<MODE, GATHER, WT, MANT, SPLIT>),
               static_cast<int>(lds_bytes_max<WT>()));
    const int klen = g.kd / ks;
    size_t extra = 0;
    if (WT == kWtMxfp4) extra = 256 * static_cast<size_t>(klen / 32);
    if (WT == kWtFp8 && klen / 128 > 64)
        extra = fp8_code_bytes(klen / 128) + (MANT ? 2 * sizeof(float) * static_cast<size_t>(klen / 128) : 0);
    const size_t lds = kStages * stage_bytes<WT>() + extra;
    if (SPLIT) {
        GroupedGemmArgs gs = g;
        gs.k_slices = ks;
        gemm_prefill<MODE, GATHER, WT, MANT, SPLIT><<<blocks, 256, lds, st>>>(gs);
    } else {
        gemm_prefill<MODE, GATHER, WT, MANT, SPLIT><<<blocks, 256, lds, st>>>(g);
    }
}

template <int WT, bool MANT>
static void launch_prefill_dtype(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, int blocks, int ks) {
    // split K only for a single weight set (rows in token order, no gather); the grid
    // enumerates every (row tile bound, column tile, slice)
    if (ks > 1) {
        const int ncol = (mode == kGateUp) ? 128 : 256;
        const int nb = g.max_tiles * (g.n_out / ncol) * ks;
        if (mode == kGateUp) launch_prefill_inst<kGateUp, false, WT, MANT, true>(st, g, nb, ks);
        else launch_prefill_inst<kDown, false, WT, MANT, true>(st, g, nb, ks);
    } else if (mode == kGateUp) {
        if (g.gather) launch_prefill_inst<kGateUp, true, WT, MANT, false>(st, g, blocks, 1);
        else launch_prefill_inst<kGateUp, false, WT, MANT, false>(st, g, blocks, 1);
    } else {
        if (g.gather) launch_prefill_inst<kDown, true, WT, MANT, false>(st, g, blocks, 1);
        else launch_prefill_inst<kDown, false, WT, MANT, false>(st, g, blocks, 1);
    }
}

int prefill_k_split(GemmMode mode, const GroupedGemmArgs& g, PrefillWeights wt) {
    if (!g.part || g.gather) return 1;
    const int ncol = (mode == kGateUp) ? 128 : 256;
    const int64_t out_elems = static_cast<int64_t>(g.max_rows) * g.n_out * (mode == kGateUp ? 2 : 1);
    int ks = decode_k_split(static_cast<int64_t>(g.max_tiles) * (g.n_out / ncol), g.kd, 512, out_elems, g.part_cap);
    // MXFP4: a slice's weight scales must fit in LDS
    if (wt == PrefillWeights::kMxfp4)
        while (g.kd / ks > kMxfp4PrefillMaxKd) ks *= 2;
    return ks;
}

int launch_gemm_prefill(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, PrefillWeights wt) {
    if (g.max_tiles == 0) return 1;
    const int ncol = (mode == kGateUp) ? 128 : 256;
    // every (row tile, column tile) of whole groups of group_m row tiles, in whole XCD chunks
    const int64_t groups = (g.max_tiles + g.group_m - 1) / g.group_m;
    const int blocks = static_cast<int>((groups * g.group_m * (g.n_out / ncol) + 255) / 256 * 256);
    const int ks = prefill_k_split(mode, g, wt);
    if (wt == PrefillWeights::kFp8 && g.w_scale_pow2) launch_prefill_dtype<kWtFp8, false>(st, mode, g, blocks, ks);
    else if (wt == PrefillWeights::kFp8) launch_prefill_dtype<kWtFp8, true>(st, mode, g, blocks, ks);
    else if (wt == PrefillWeights::kMxfp4) launch_prefill_dtype<kWtMxfp4, false>(st, mode, g, blocks, ks);
    else launch_prefill_dtype<kWtBf16, false>(st, mode, g, blocks, ks);
    return ks;
}

}  // namespace beam
