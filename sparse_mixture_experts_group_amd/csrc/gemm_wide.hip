// Grouped expert GEMMs for many rows per expert with BF16 or FP8 (OCP E4M3FN, one FP32
// scale per 128 x 128 block, E4M3 activations with row scales) weights: LDS-tiled MFMA
// GEMM whose K stages hold 128 bytes of every operand row.
//
// SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of Experts: 256 experts, 8
// routed per token"; FP32 SwiGLU product per the "Residual stream" section):
//   gate/up:  h[r, j] = SiLU(a_r . Wg[j]) * (a_r . Wu[j])   (a_r gathered by token)
//   down:     y[r, n] = h_r . Wd[n]
// Tiles, wave roles and block order are those of the 64-byte-stage kernel in
// gemm_prefill.hip (which serves the other cases): 256 x 256 output tiles of one expert,
// 4 waves of 128 x 128 as 4 x 4 MFMA tiles of 32 x 32, gate and up rows of the same
// columns in one tile so the SwiGLU is applied in registers.  The MFMAs take the weights
// as their A operand and so compute the transposed tile, whose lane layout lets the
// epilogue (tile_epilogue.cuh) store 4 columns of a row at a time.
//
// Why 128-byte stages: a direct global->LDS load moves 16 bytes per lane; with 64-byte
// row pieces every request covers half an L2 line, and measured on gfx950 the L2 then
// delivers 16-19 TB/s to LDS against 30-32 TB/s for 128-byte row pieces (panels
// resident in L2), which is what bounds the 64-byte-stage kernel where activation tiles
// and shared weight panels come from L2.  A stage is 32 KB of activations (256 rows x
// 128 bytes) and 32 KB of weights; the 160 KB of LDS hold two activation slots and three
// weight slots, so while stage j is computed the activations of stage j + 1 and the
// weights of stages j + 1 and j + 2 (the HBM stream) are in flight.  Measured on the
// Beam layer against the 64-byte-stage kernel: 4096 tokens (BF16) gate/up 2.53 against
// 2.83 ms, 32768 skewed tokens 13.67 against 13.71, 8192 tokens with FP8 weights 2.55
// against 2.72.
//
// Load issue: a 16-byte-per-lane load holds the wave's issue for many cycles, so a burst
// of them leaves the matrix pipe idle (counters: MFMA busy 55% of the time with the 16
// loads of a stage issued two per MFMA, 77% with none).  The loads are buffer loads
// (32-bit lane offsets fixed per block, the stage advance in a scalar offset) spread
// over the MFMAs of the whole stage: skewed 32768 tokens gate/up 13.46 -> 12.11 ms,
// dense MLP at 4096 tokens 2.41 -> 2.19 ms per step.
#include "common.cuh"
#include "kernels.h"
#include "tile_epilogue.cuh"

namespace beam {

namespace {
constexpr int kWideRowBytes = 128;               // K bytes of an operand row per stage
constexpr int kWideOpBytes = 256 * kWideRowBytes;     // one operand (256 rows) of one stage
constexpr int kWideASlots = 2, kWideBSlots = 3;
constexpr size_t kWideLds = (kWideASlots + kWideBSlots) * static_cast<size_t>(kWideOpBytes);
static_assert(kWideLds <= 160 * 1024, "LDS budget");
static_assert(kWideLds >= wide_epilogue_lds(kDown) && kWideLds >= wide_epilogue_lds(kGateUp), "epilogue staging");

// 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 7): the 16 consecutive rows one
// fragment read serves per LDS cycle (same chunk) fill both halves of the 256-byte bank
// period with 8 distinct slots each, i.e. all 64 banks.
__device__ __forceinline__ int wide_offset(int row, int chunk) {
    return row * kWideRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Byte offset inside a row's 128-byte K piece of the chunk lane `lane` moves in a DMA
// instruction covering rows base .. base + 7 (base a multiple of 8, `odd` = bit 3 of
// base): lane i lands in row base + i / 8, slot i % 8.
__device__ __forceinline__ int wide_dma_chunk(int lane, int odd) {
    return ((lane & 7) ^ (((lane >> 4) + 4 * odd) & 7)) << 4;
}

constexpr int kUnitScale = 0x7f;                 // E8M0 code of 2^0

// Waves per block.  With 4 the accumulators of a 128 x 128 wave tile fill the AGPRs, and
// the significand fold of FP8 blocks with general scales (MANT) would need three vector
// instructions per accumulator (AGPR -> VGPR, multiply, back) and spill; with 8 waves of
// 64 x 128 the accumulators sit in VGPRs and the fold is one multiply each, which runs
// beside the MFMAs.  Measured on the Beam layer (one MI355X): FP8 sublayer at 8192 tokens
// with amax / 448 block scales 9.27 ms (4 waves) against 4.11 ms (8); for BF16 and
// power-of-two scales the two are within 2-3% (skewed 32768 tokens 20.74 / 20.56 ms,
// 4096 tokens 4.29 / 4.32, FP8 power-of-two sublayer 3.89 / 3.99), so those keep 4.
template <bool MANT> constexpr int wide_waves() { return MANT ? 8 : 4; }

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Fragments of one MFMA K step for one wave: BF16 - 16 K values (8 per lane); FP8 - 64 K
// values (32 per lane).
template <bool FP8> struct StepFrags;
template <> struct StepFrags<false> { bf16x8 a[4]; bf16x8 b[4]; };
template <> struct StepFrags<true> { i32x8 a[4]; i32x8 b[4]; };
}  // namespace

// Pipeline per stage kt (KS MFMA K steps: 4 of 16 for BF16, 2 of 64 for FP8), fragments double
// buffered in registers: K steps 0 .. KS-2 run their MFMAs while reading the next step's
// fragments from the stage's slots and loading a share of the weights of stage kt + 2
// into the slot stage kt - 1 drained; before the last step every wave waits until stage
// kt + 1 has landed (only the weight loads of stage kt + 2 may still be in flight) and
// meets the others, then runs the last step's MFMAs while reading stage kt + 1's first
// fragments and loading the activations of stage kt + 2 into the slot stage kt drained.
// FP8: one 128 x 128 scale block per stage, at most 64 per reduction (a lane of a
// register each).  The scaled MFMA applies the exponent of the block's FP32 scale (its
// E8M0 code) to the weights.  MANT (scales that are not all powers of two): the
// significand m in [1, 2) of each block scale is folded on the vector ALU by keeping the
// accumulators in units of the current block's m -- before the MFMAs of K block kb they
// are multiplied by m[kb-1] / m[kb] (1 for the first block), after the last block by
// m[last] -- one multiply per accumulator and stage, no second set of accumulators.
//
// SPLIT: as in gemm_prefill.hip, the GEMMs of a single weight set split K into
// g.k_slices slices (FP32 partial sums) over a flat block order.
// WAVES: 4 waves of 128 x 128 (one per SIMD), or 8 waves of 64 x 128 (two per SIMD, so
// one wave's MFMAs run while the other waits at a barrier or for its loads).  The WR =
// WAVES / 2 wave rows take the 32-row MFMA tiles in turn: wave row wm owns tiles wm,
// wm + WR, ...
template <int MODE, bool GATHER, bool FP8, bool MANT, bool SPLIT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_wide(GroupedGemmArgs g) {
    static_assert(FP8 || !MANT, "block-scale significands are an FP8 feature");
    static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
    constexpr int WR = WAVES / 2;                       // wave rows
    constexpr int BM = kPrefillBM, BN = 256, MI = 8 / WR, NI = 4;
    constexpr int NB = BN / WAVES;                      // weight rows each wave moves per stage
    constexpr int JB = NB / 8;                          // its direct-to-LDS loads per stage
    constexpr int EB = FP8 ? 1 : 2;                     // bytes per element (A and B)
    constexpr int BK = kWideRowBytes / EB;              // K per stage
    constexpr int KS = FP8 ? 2 : 4;                     // MFMA K steps per stage
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
    const int64_t krow = static_cast<int64_t>(g.kd) * EB;        // bytes per weight row
    const int klen = SPLIT ? g.kd / g.k_slices : g.kd;           // K slice of this block
    const int kbeg = SPLIT ? kz * klen : 0;

    // MFMA row tiles of this wave that hold rows of the expert (wave-uniform; a prefix of
    // the wave's tiles): the others skip their loads, LDS reads and MFMAs.
    const int ntiles = (rows + 31) / 32;
    const int mvalid = __builtin_amdgcn_readfirstlane(min(MI, max(0, (ntiles - wm + WR - 1) / WR)));

    // Direct-to-LDS assignment, 8 rows x 128 bytes per wave instruction.  A: wave (wm, wn)
    // moves rows (wm + WR i) * 32 + 16 wn + 8 h + lane / 8 (h < 2) of each of its live row
    // tiles i, the rows the pair (wm, 0), (wm, 1) reads; rows past the expert's end
    // re-load its last row (never read back).  B: wave w moves rows w * NB + 8 j + lane / 8
    // (j < JB; for gate/up the first half of the waves move gate rows, the rest up rows).
    // Addresses are block-uniform bases plus 32-bit lane offsets (the launcher checks
    // that the activation rows span less than 4 GB; one expert's weights always do).
    const int dr = lane >> 3;
    const uint8_t* abase = static_cast<const uint8_t*>(g.a) + static_cast<int64_t>(kbeg) * EB;
    uint32_t aoff[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rr = min((wm + WR * i) * 32 + 16 * wn + 8 * h + dr, rows - 1);
            const int64_t arow = GATHER ? g.pair_of_row[row0 + rr] / g.topk : static_cast<int64_t>(row0 + rr);
            aoff[i][h] = static_cast<uint32_t>(arow * g.lda * EB) + wide_dma_chunk(lane, h);
        }
    auto weight_row = [&](int r) -> int {                // block row r (0..255) -> weight row
        if (MODE == kGateUp) return (r < BN / 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        return c0 + r;
    };
    const uint8_t* bbase = static_cast<const uint8_t*>(g.w) + static_cast<int64_t>(e) * nw * krow +
                           static_cast<int64_t>(kbeg) * EB;
    const uint32_t boff = static_cast<uint32_t>(weight_row(wave * NB + dr) * krow);
    const uint32_t bch0 = wide_dma_chunk(lane, 0), bch1 = wide_dma_chunk(lane, 1);
    const uint32_t bstep = static_cast<uint32_t>(8 * krow);   // bytes between B rows j and j + 1
    const __amdgpu_buffer_rsrc_t rsrc_a = buffer_rsrc(abase, (g.a_rows * g.lda - kbeg) * EB);
    const __amdgpu_buffer_rsrc_t rsrc_b = buffer_rsrc(bbase, nw * krow - static_cast<int64_t>(kbeg) * EB);

    // FP8 weight-scale exponents: lane l holds the E8M0 code of K block l of the slice
    // (gate-column block in s_lo, up-column block in s_hi for gate/up; this wave's column
    // block for down).  MANT: lane l also holds the ratio m[l-1] / m[l] of the blocks'
    // significands (q_lo, q_hi; 1 for l = 0), and m_end_* is the last block's.
    int s_lo = kUnitScale, s_hi = kUnitScale;
    float q_lo = 1.0f, q_hi = 1.0f, m_end_lo = 1.0f, m_end_hi = 1.0f;
    if constexpr (FP8) {
        const int kb_all = g.kd / 128, kb_n = klen / 128;
        const float* wsc = static_cast<const float*>(g.w_scale) + kbeg / 128;
        const float* r_lo;
        const float* r_hi;
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
    for (int i = 0; i < MI; ++i) arow_l[i] = (wm + WR * i) * 32 + l32;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        brow_l[i] = (MODE == kGateUp) ? ((i < 2) ? wn * 64 + i * 32 : BN / 2 + wn * 64 + (i - 2) * 32) + l32
                                      : wn * 128 + i * 32 + l32;
    }
    const int nk = klen / BK;          // slices are multiples of BK

    auto k_loop = [&](auto mv_tag) {
        constexpr int MV = decltype(mv_tag)::value;
        constexpr int NM = MV * NI;                      // MFMAs per K step
        constexpr int NR = MV == 0 ? 0 : (FP8 ? 2 : 1) * (MV + NI);   // LDS reads per K step
        auto dma_a = [&](int slot, int kt) {            // activations of stage kt
            uint8_t* As = smem + slot * kWideOpBytes;
            const int ks = kt * kWideRowBytes;
#pragma unroll
            for (int i = 0; i < MI; ++i)
                if (i < MV) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        lds_dma16_buf(rsrc_a, As + ((wm + WR * i) * 32 + 16 * wn + 8 * h) * kWideRowBytes, aoff[i][h], ks);
                }
        };
        // weights of stage kt: loads J0 .. J1 - 1 of the wave's JB
        auto dma_b = [&](int slot, int kt, auto j0_tag, auto j1_tag) {
            constexpr int J0 = decltype(j0_tag)::value, J1 = decltype(j1_tag)::value;
            uint8_t* Bs = smem + (kWideASlots + slot) * kWideOpBytes;
            const int ks = kt * kWideRowBytes;
#pragma unroll
            for (int j = J0; j < J1; ++j)
                lds_dma16_buf(rsrc_b, Bs + (wave * NB + 8 * j) * kWideRowBytes, boff + j * bstep + ((j & 1) ? bch1 : bch0),
                              ks);
        };
        auto rd = [&](const uint8_t* T, int row, int c) {
            return *reinterpret_cast<const u32x4*>(T + wide_offset(row, c));
        };
        // fragments of K step s of a stage whose operands are in slots aslot, bslot
        auto load_frags = [&](StepFrags<FP8>& f, int aslot, int bslot, int s) {
            const uint8_t* As = smem + aslot * kWideOpBytes;
            const uint8_t* Bs = smem + (kWideASlots + bslot) * kWideOpBytes;
            if constexpr (FP8) {
                // 32 bytes per lane: K values 64 s + 32 lh .. + 31 = chunks 4 s + 2 lh, + 1
                const int c = 4 * s + 2 * lh;
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) f.a[mi] = join8(rd(As, arow_l[mi], c), rd(As, arow_l[mi], c + 1));
                if (MV > 0) {
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) f.b[ni] = join8(rd(Bs, brow_l[ni], c), rd(Bs, brow_l[ni], c + 1));
                }
            } else {
                // 16 bytes per lane: K values 16 s + 8 lh .. + 7 = chunk 2 s + lh
                const int c = 2 * s + lh;
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) f.a[mi] = __builtin_bit_cast(bf16x8, rd(As, arow_l[mi], c));
                if (MV > 0) {
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) f.b[ni] = __builtin_bit_cast(bf16x8, rd(Bs, brow_l[ni], c));
                }
            }
        };
        // first: the stage's first K step, where MANT moves the accumulators into the units
        // of this stage's block-scale significands
        auto mfma_step = [&](const StepFrags<FP8>& f, int kt, auto first_tag) {
            if constexpr (FP8) {
                // the stage's 128-wide K block is kt (< 64)
                const int sc_lo = __builtin_amdgcn_readlane(s_lo, kt);
                const int sc_hi = __builtin_amdgcn_readlane(s_hi, kt);
                if constexpr (MANT && decltype(first_tag)::value) {
                    // into the units of this block's significands, one tile at a time right
                    // before its MFMA (so few values are in flight between the register files)
                    const float r_lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q_lo), kt));
                    const float r_hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q_hi), kt));
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        if (mi < MV) {
#pragma unroll
                            for (int ni = 0; ni < NI; ++ni) {
                                const float r = (MODE == kGateUp && ni >= 2) ? r_hi : r_lo;
#pragma unroll
                                for (int i = 0; i < 16; ++i) acc[mi][ni][i] *= r;
                                const int sb = (MODE == kGateUp && ni >= 2) ? sc_hi : sc_lo;
                                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0, sb, 0, kUnitScale);
                                __builtin_amdgcn_sched_barrier(0);
                            }
                        }
                } else {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        if (mi < MV) {
#pragma unroll
                            for (int ni = 0; ni < NI; ++ni) {
                                const int sb = (MODE == kGateUp && ni >= 2) ? sc_hi : sc_lo;
                                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0, sb, 0, kUnitScale);
                            }
                        }
                }
            } else {
                (void)kt;
                (void)first_tag;
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    if (mi < MV) {
#pragma unroll
                        for (int ni = 0; ni < NI; ++ni)
                            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
                    }
            }
        };

        StepFrags<FP8> f0, f1;
        // The loop body is branch-free (a branch would split the fragment registers into
        // copies at its join): stage indices past the end are clamped, and the last
        // iterations re-load the last stage into slots nothing reads any more, so every
        // stage issues the same loads and every wait count is fixed.
        // Prologue order: A0 B0 A1 B1; wait for stage 0 (A0, B0).  Issue order in the
        // loop: B(kt + 2) during the first K steps of stage kt, A(kt + 2) in its last.
        using I0 = std::integral_constant<int, 0>;
        using IJ = std::integral_constant<int, JB>;
        dma_a(0, 0);
        dma_b(0, 0, I0{}, IJ{});
        dma_a(1, min(1, nk - 1));
        dma_b(1, min(1, nk - 1), I0{}, IJ{});
        wait_lds_dma<2 * MV + JB>();
        lds_pipeline_barrier();
        load_frags(f0, 0, 0, 0);
        int bslot = 0;                                   // weight slot of stage kt (kt % 3)
        for (int kt = 0; kt < nk; ++kt) {
            const int aslot = kt & 1;
            const int bnext = (bslot == kWideBSlots - 1) ? 0 : bslot + 1;
            const int bfree = (bslot == 0) ? kWideBSlots - 1 : bslot - 1;   // stage kt - 1's slot
            // K steps 0 .. KS-2 (KS is even, so the buffers alternate statically): the next
            // step's fragments, then a share of the weights of stage kt + 2
            static_for<0, KS - 1>([&](auto s_tag) {
                constexpr int s = decltype(s_tag)::value;
                constexpr int j0 = (JB * s) / (KS - 1), j1 = (JB * (s + 1)) / (KS - 1);
                StepFrags<FP8>& cur = (s & 1) ? f1 : f0;
                StepFrags<FP8>& nxt = (s & 1) ? f0 : f1;
                __builtin_amdgcn_sched_barrier(0);
                mfma_step(cur, kt, std::integral_constant<bool, s == 0>{});
                load_frags(nxt, aslot, bslot, s + 1);
                dma_b(bfree, min(kt + 2, nk - 1), std::integral_constant<int, j0>{}, std::integral_constant<int, j1>{});
                sched_reads_then_loads<NM, NR, j1 - j0>();
                __builtin_amdgcn_sched_barrier(0);
            });
            // last K step.  Issue order so far ends ... A(kt+1), B(kt+2): stage kt + 1 has
            // landed once at most the JB weight loads of stage kt + 2 are in flight.
            wait_lds_dma<JB>();
            lds_pipeline_barrier();
            __builtin_amdgcn_sched_barrier(0);
            mfma_step(f1, kt, std::false_type{});
            load_frags(f0, aslot ^ 1, bnext, 0);
            dma_a(aslot, min(kt + 2, nk - 1));           // into the slot stage kt drained
            sched_reads_then_loads<NM, NR, 2 * MV>();
            __builtin_amdgcn_sched_barrier(0);
            bslot = bnext;
        }
        wait_lds_dma<0>();      // the tail's re-loads land before the block's LDS is released
    };
    dispatch_row_tiles<MI>(mvalid, k_loop);
    if constexpr (MANT) {
        // from the units of the last block's significand back to the block scales
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const float m = (MODE == kGateUp && ni >= 2) ? m_end_hi : m_end_lo;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mi][ni][i] *= m;
            }
    }

    // down: 256-byte row segments per wave, staged through LDS for whole-row stores;
    // gate/up (128-byte segments) and FP32 partial sums: stored from the registers
    if constexpr (SPLIT || MODE == kGateUp) {
        store_wide_tile<MODE, GATHER, FP8, SPLIT, WR>(g, acc, rows, row0, c0, wm, wn, lane, kz);
    } else {
        __syncthreads();                 // every wave is out of its K loop: the LDS is free
        store_wide_tile_bf16<MODE, GATHER, FP8, WR>(g, acc, rows, row0, c0, wm, wn, wave, lane, smem);
    }
}

template <int MODE, bool GATHER, bool FP8, bool MANT, bool SPLIT>
static void launch_wide_inst(hipStream_t st, const GroupedGemmArgs& g, int blocks, int ks) {
    constexpr int W = wide_waves<MANT>();
    lds_opt_in(reinterpret_cast<const void*>(&gemm_wide<MODE, GATHER, FP8, MANT, SPLIT, W>), static_cast<int>(kWideLds));
    const size_t lds = kWideLds;
    if (SPLIT) {
        GroupedGemmArgs gs = g;
        gs.k_slices = ks;
        gemm_wide<MODE, GATHER, FP8, MANT, SPLIT, W><<<blocks, 64 * W, lds, st>>>(gs);
    } else {
        gemm_wide<MODE, GATHER, FP8, MANT, SPLIT, W><<<blocks, 64 * W, lds, st>>>(g);
    }
}

template <bool FP8, bool MANT>
static void launch_wide_modes(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, int blocks, int ks) {
    // split K only for a single weight set (rows in token order, no gather); the grid
    // enumerates every (row tile bound, column tile, slice)
    if (ks > 1) {
        const int ncol = (mode == kGateUp) ? 128 : 256;
        const int nb = g.max_tiles * (g.n_out / ncol) * ks;
        if (mode == kGateUp) launch_wide_inst<kGateUp, false, FP8, MANT, true>(st, g, nb, ks);
        else launch_wide_inst<kDown, false, FP8, MANT, true>(st, g, nb, ks);
    } else if (mode == kGateUp) {
        if (g.gather) launch_wide_inst<kGateUp, true, FP8, MANT, false>(st, g, blocks, 1);
        else launch_wide_inst<kGateUp, false, FP8, MANT, false>(st, g, blocks, 1);
    } else {
        if (g.gather) launch_wide_inst<kDown, true, FP8, MANT, false>(st, g, blocks, 1);
        else launch_wide_inst<kDown, false, FP8, MANT, false>(st, g, blocks, 1);
    }
}

int launch_gemm_wide(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, bool fp8) {
    if (g.max_tiles == 0) return 1;
    const int ncol = (mode == kGateUp) ? 128 : 256;
    // every (row tile, column tile) of whole groups of group_m row tiles, in whole XCD chunks
    const int64_t groups = (g.max_tiles + g.group_m - 1) / g.group_m;
    const int blocks = static_cast<int>((groups * g.group_m * (g.n_out / ncol) + 255) / 256 * 256);
    const int ks = prefill_k_split(mode, g, fp8 ? PrefillWeights::kFp8 : PrefillWeights::kBf16);
    if (!fp8) launch_wide_modes<false, false>(st, mode, g, blocks, ks);
    else if (g.w_scale_pow2) launch_wide_modes<true, false>(st, mode, g, blocks, ks);
    else launch_wide_modes<true, true>(st, mode, g, blocks, ks);
    return ks;
}

}  // namespace beam
