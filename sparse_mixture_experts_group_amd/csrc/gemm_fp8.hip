// FP8 (OCP E4M3FN) grouped expert GEMMs on the gfx950 f8f6f4 MFMA, FP32 accumulation.
//
// Weights carry one FP32 scale per 128 x 128 tile (value = code * scale); activations
// are quantised on the GPU with one FP32 scale per row (amax / 448).  The reduction is
// split into 128-wide K blocks, one weight-scale block each: the block's partial
// product is formed on the matrix core with unit hardware scales and folded into the
// FP32 accumulator with one fma by the (wave-uniform) weight scale; the row scale is
// applied once in the epilogue.  Same two shapes and the same SwiGLU fusion as the
// BF16 kernels (decode: weight streaming with v_mfma_scale_f32_16x16x128_f8f6f4;
// prefill: BM x 256 LDS tiles with v_mfma_scale_f32_32x32x64_f8f6f4).
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
// prefill: 256 x 256 block tile, 128 x 128 per wave, K blocks of 128 bytes via LDS
// ---------------------------------------------------------------------------
// Same tiling and LDS layout as the BF16 prefill kernel (a 128-entry FP8 K block is the
// 128-byte row of one LDS tile).  Per K block and per 32 x 32 output tile, two
// v_mfma_scale_f32_32x32x64_f8f6f4 form the block's partial product in a temporary,
// which is folded into the accumulator with one fma by the weight-tile scale (uniform
// over the wave's columns of one weight-scale block).
constexpr int kF8BK = 128;
template <int BM> constexpr int f8_stage_bytes() { return (BM + kTileRows) * kTileRowBytes; }
template <int BM> constexpr size_t f8_lds_bytes() { return 2 * f8_stage_bytes<BM>(); }

// BM = 256: each wave owns 128 rows (4 MFMA row tiles); BM = 128: 64 rows (2 row tiles).
template <int MODE, bool GATHER, int BM>
__global__ __launch_bounds__(256) void gemm_fp8_prefill(GroupedGemmArgs g) {
    constexpr int BN = 256, BK = kF8BK, MI = BM / 64, WROWS = BM / 2;
    constexpr int kF8StageBytes = f8_stage_bytes<BM>();
    static_assert((BM == 256 || BM == 128) && BN == kTileRows && BK == kTileRowBytes, "tile geometry");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];
    constexpr int NCOL = (MODE == kGateUp) ? BN / 2 : BN;
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
    const int kb_n = g.kd / 128;

    const int lr = lane >> 3, ls = lane & 7;
    constexpr int AJ = BM / 32;
    const uint8_t* ag[AJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
        const int r = wave * (BM / 4) + j * 8 + lr;
        const int rr = min(r, rows - 1);
        const int64_t arow = GATHER ? g.pair_of_row[row0 + rr] / g.topk : static_cast<int64_t>(row0 + rr);
        ag[j] = static_cast<const uint8_t*>(g.a) + arow * g.lda + ((ls ^ ((r >> 1) & 7)) << 4);
    }
    const uint8_t* bg;
    {
        const int r = wave * 64 + lr;
        int64_t wrow;
        if (MODE == kGateUp) wrow = (wave < 2) ? c0 + r : g.n_out + c0 + (r - BN / 2);
        else wrow = c0 + r;
        bg = static_cast<const uint8_t*>(g.w) + (static_cast<int64_t>(e) * nw + wrow) * g.kd;
    }
    const int64_t bstep = 8 * static_cast<int64_t>(g.kd);
    const int boff_lane[2] = {(ls ^ (lr >> 1)) << 4, (ls ^ (4 + (lr >> 1))) << 4};
    auto dma = [&](int stage, int k0) {
        uint8_t* As = smem8 + stage * kF8StageBytes;
        uint8_t* Bs = As + BM * kTileRowBytes;
#pragma unroll
        for (int j = 0; j < AJ; ++j)
            lds_dma16(ag[j] + k0, As + (wave * (BM / 4) + j * 8) * kTileRowBytes);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            lds_dma16(bg + j * bstep + k0 + boff_lane[j & 1], Bs + (wave * 64 + j * 8) * kTileRowBytes);
    };
    // weight-scale rows: gate / up blocks (gate-up) or this wave's column block (down)
    const float* sw0;
    const float* sw1;
    if (MODE == kGateUp) {
        sw0 = g.w_scale + (static_cast<int64_t>(e) * (nw / 128) + c0 / 128) * kb_n;
        sw1 = g.w_scale + (static_cast<int64_t>(e) * (nw / 128) + (g.n_out + c0) / 128) * kb_n;
    } else {
        sw0 = g.w_scale + (static_cast<int64_t>(e) * (nw / 128) + (c0 + wn * 128) / 128) * kb_n;
        sw1 = sw0;
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
    for (int i = 0; i < MI; ++i) arow_l[i] = wm * WROWS + i * 32 + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        brow_l[i] = (MODE == kGateUp) ? ((i < 2) ? wn * 64 + i * 32 : BN / 2 + wn * 64 + (i - 2) * 32) + l32
                                      : wn * 128 + i * 32 + l32;
    }
    // 32-row MFMA tiles of this wave that hold rows of the expert (wave-uniform): the
    // others (padding of an expert's last tile) skip their LDS reads, MFMAs and folds.
    const int mvalid = __builtin_amdgcn_readfirstlane(min(MI, max(0, (rows - wm * WROWS + 31) / 32)));
    // fragment of K half hk: 32 bytes = chunks 4 hk + 2 lh and 4 hk + 2 lh + 1 of the row
    auto frag = [&](const uint8_t* T, int row, int hk) {
        const int c = hk * 4 + lh * 2;
        return join(*reinterpret_cast<const u32x4*>(T + tile_offset(row, c)),
                    *reinterpret_cast<const u32x4*>(T + tile_offset(row, c + 1)));
    };

    // One K block (128 bytes) from LDS stage `stage`, as 2*MI groups of (one row tile,
    // two column tiles).  The 4 MFMAs of group q go to temporary set q & 1 while the 32
    // FMAs folding group q - 1 (scale of its weight block) run: MFMA and VALU overlap,
    // and each fold reads results issued a whole group earlier.
    auto k_block = [&](auto mv_tag, int stage, float s0, float s1) {
        constexpr int MV = decltype(mv_tag)::value;
        const uint8_t* As = smem8 + stage * kF8StageBytes;
        const uint8_t* Bs = As + BM * kTileRowBytes;
        i32x8 bfm[2][4];
#pragma unroll
        for (int hk = 0; hk < 2; ++hk)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) bfm[hk][ni] = frag(Bs, brow_l[ni], hk);
        i32x8 af[2][2];
        f32x16 t[2][2];
        constexpr int NG = 2 * MI;
#pragma unroll
        for (int q = 0; q <= NG; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            if (q < NG && (q >> 1) < MV) {
                const int mi = q >> 1, np = q & 1;
                if (np == 0) {
#pragma unroll
                    for (int hk = 0; hk < 2; ++hk) af[mi & 1][hk] = frag(As, arow_l[mi], hk);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    f32x16 z = {};
                    t[q & 1][j] = mfma32_fp8(af[mi & 1][0], bfm[0][2 * np + j], z);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    t[q & 1][j] = mfma32_fp8(af[mi & 1][1], bfm[1][2 * np + j], t[q & 1][j]);
            }
            if (q > 0 && ((q - 1) >> 1) < MV) {
                const int p = q - 1, mi = p >> 1, np = p & 1;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int ni = 2 * np + j;
                    const float sc = (MODE == kGateUp) ? (ni < 2 ? s0 : s1) : s0;
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[mi][ni][i] = fmaf(t[p & 1][j][i], sc, acc[mi][ni][i]);
                }
            }
            if (q < NG && q > 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    constexpr int PER = AJ + 8;       // direct-to-LDS loads per K block per wave
    const int nk = g.kd / BK;
    dma(0, 0);
    wait_lds_dma<0>();
    lds_pipeline_barrier();
    // two-stage pipeline, branch-free body: the last iteration re-loads the last block
    // into the idle stage (clamped index), which nothing reads
    // The K loop is instantiated per count of live row tiles, so no instance tests them.
    auto k_loop = [&](auto mv_tag) {
        for (int kt = 0; kt < nk; ++kt) {
            const int stage = kt & 1;
            __builtin_amdgcn_sched_barrier(0);
            dma(stage ^ 1, min(kt + 1, nk - 1) * BK);
            k_block(mv_tag, stage, sw0[kt], sw1[kt]);
            wait_lds_dma<0>();
            lds_pipeline_barrier();
        }
    };
    dispatch_row_tiles<MI>(mvalid, k_loop);
    (void)PER;

    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * WROWS + mi * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
            if (m >= rows) continue;
            const int64_t ar = GATHER ? g.pair_of_row[row0 + m] / g.topk : static_cast<int64_t>(row0 + m);
            const float sa = g.a_scale[ar];
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

template <int MODE, bool GATHER, int BM>
void launch_fp8_prefill_inst(hipStream_t st, const GroupedGemmArgs& g, int blocks) {
    static bool attr_set = false;     // the LDS opt-in is per kernel, set on first use
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_fp8_prefill<MODE, GATHER, BM>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(f8_lds_bytes<BM>()));
        attr_set = true;
    }
    gemm_fp8_prefill<MODE, GATHER, BM><<<blocks, 256, f8_lds_bytes<BM>(), st>>>(g);
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
    const int ncol = (mode == kGateUp) ? 128 : 256;
    const int blocks = (g.max_tiles * (g.n_out / ncol) + 255) / 256 * 256;   // whole XCD chunks
    const bool small = g.bm == kPrefillBMMin;
    if (mode == kGateUp) {
        if (g.gather) {
            if (small) launch_fp8_prefill_inst<kGateUp, true, kPrefillBMMin>(st, g, blocks);
            else launch_fp8_prefill_inst<kGateUp, true, kPrefillBMMax>(st, g, blocks);
        } else {
            if (small) launch_fp8_prefill_inst<kGateUp, false, kPrefillBMMin>(st, g, blocks);
            else launch_fp8_prefill_inst<kGateUp, false, kPrefillBMMax>(st, g, blocks);
        }
    } else {
        if (g.gather) {
            if (small) launch_fp8_prefill_inst<kDown, true, kPrefillBMMin>(st, g, blocks);
            else launch_fp8_prefill_inst<kDown, true, kPrefillBMMax>(st, g, blocks);
        } else {
            if (small) launch_fp8_prefill_inst<kDown, false, kPrefillBMMin>(st, g, blocks);
            else launch_fp8_prefill_inst<kDown, false, kPrefillBMMax>(st, g, blocks);
        }
    }
}

}  // namespace beam
