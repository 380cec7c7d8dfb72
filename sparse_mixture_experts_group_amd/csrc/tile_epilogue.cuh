// Epilogue of the LDS-tiled expert GEMMs whose MFMAs compute the transposed wave tile
// (weights as the A operand, activations as B; MI row tiles of 32 x 128 columns, the WR
// wave rows taking row tiles in turn): for row tile mi of the wave, lane (l32 = lane % 32,
// lh = lane / 32) holds token row (wm + WR mi) * 32 + l32 and, in
// group q of 8 columns of each 32-column MFMA tile ni, the 4 consecutive columns
// 8 q + 4 lh .. + 3 (accumulator entries 4 q .. 4 q + 3).  So a lane tests its row once,
// reads its row scale once and stores 4 columns at a time.
//
// gate/up (tiles 0-1 gate columns, 2-3 the up columns of the same outputs): the SwiGLU
// product SiLU(g) * u in FP32, stored as BF16; down: the sums as BF16.  SPLIT: FP32
// partial sums of K slice kz (gate then up sums per row for gate/up).
#pragma once
#include "common.cuh"
#include "kernels.h"

namespace beam {

// BF16 outputs through LDS (`stage`: the block's LDS, free once every wave has left
// its K loop and the block has met): each wave writes its 32 MI rows x NC columns with
// 8-byte writes (row pitch skewed by 8 bytes so the 32 rows of one write spread over the
// banks), then reads them back 16 bytes per lane, NC / 8 lanes per row, and stores whole
// row segments.
// Bytes of LDS the BF16 epilogue stages through (the block's 512 wave rows: 4 waves x 128
// rows, or 8 x 64).
constexpr int wide_epilogue_pitch(int mode) { return (mode == kGateUp ? 64 : 128) * 2 + 8; }
constexpr size_t wide_epilogue_lds(int mode) { return 4 * 128 * static_cast<size_t>(wide_epilogue_pitch(mode)); }

template <int MODE, bool GATHER, bool SCALED, int WR, int MI, int NI>
__device__ __forceinline__ void store_wide_tile_bf16(const GroupedGemmArgs& g, const f32x16 (&acc)[MI][NI],
                                                     int rows, int row0, int c0, int wm, int wn, int wave, int lane,
                                                     uint8_t* stage) {
    constexpr int NC = (MODE == kGateUp) ? 64 : 128;             // output columns of the wave
    constexpr int PITCH = wide_epilogue_pitch(MODE);
    static_assert(MI * WR == 8 && PITCH == NC * 2 + 8, "staging layout");
    constexpr int LPR = NC * 2 / 16;                               // lanes per row on the way out
    const int l32 = lane & 31, lh = lane >> 5;
    uint8_t* st = stage + wave * (32 * MI) * PITCH;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        float sa = 1.0f;
        if constexpr (SCALED) {
            const int m = min((wm + WR * mi) * 32 + l32, rows - 1);
            const int64_t ar = GATHER ? g.pair_of_row[row0 + m] / g.topk : static_cast<int64_t>(row0 + m);
            sa = g.a_scale[ar];
        }
        uint8_t* srow = st + (mi * 32 + l32) * PITCH;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int cq = q * 8 + lh * 4;
            uint16_t h[4];
#pragma unroll
            for (int ni = 0; ni < NC / 32; ++ni) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v = (MODE == kGateUp)
                        ? silu(acc[mi][ni][4 * q + j] * sa) * (acc[mi][ni + 2][4 * q + j] * sa)
                        : acc[mi][ni][4 * q + j] * sa;
                    h[j] = f32_to_bf16_bits(v);
                }
                *reinterpret_cast<u32x2*>(srow + (ni * 32 + cq) * 2) =
                    u32x2{h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16)};
            }
        }
    }
    // a wave's LDS operations complete in order; wait for the writes before reading back
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int it = 0; it < 32 * MI / (64 / LPR); ++it) {
        const int lr = it * (64 / LPR) + lane / LPR;              // wave row 0 .. 32 MI - 1
        const int lc = (lane % LPR) * 8;                          // first of the lane's 8 columns
        const int m = (wm + WR * (lr >> 5)) * 32 + (lr & 31);     // row of the block tile
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + lr * PITCH + lc * 2);
        if (m < rows)
            *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(row0 + m) * g.ldo + c0 + wn * NC + lc) = v;
    }
}

template <int MODE, bool GATHER, bool SCALED, bool SPLIT, int WR, int MI, int NI>
__device__ __forceinline__ void store_wide_tile(const GroupedGemmArgs& g, const f32x16 (&acc)[MI][NI], int rows,
                                                int row0, int c0, int wm, int wn, int lane, int kz) {
    const int l32 = lane & 31, lh = lane >> 5;
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int m = (wm + WR * mi) * 32 + l32;
        if (m >= rows) continue;
        float sa = 1.0f;
        if constexpr (SCALED) {
            const int64_t ar = GATHER ? g.pair_of_row[row0 + m] / g.topk : static_cast<int64_t>(row0 + m);
            sa = g.a_scale[ar];
        }
        const int64_t orow = static_cast<int64_t>(row0 + m);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int cq = q * 8 + lh * 4;               // the lane's first column in a 32-column tile
            if constexpr (SPLIT) {
                float* prow = g.part + kz * g.part_slice + orow * (MODE == kGateUp ? 2 * g.n_out : g.ldo);
                if constexpr (MODE == kGateUp) {
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const int c = c0 + wn * 64 + ni * 32 + cq;
                        f32x4 vg, vu;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            vg[j] = acc[mi][ni][4 * q + j] * sa;
                            vu[j] = acc[mi][ni + 2][4 * q + j] * sa;
                        }
                        *reinterpret_cast<f32x4*>(prow + c) = vg;
                        *reinterpret_cast<f32x4*>(prow + g.n_out + c) = vu;
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        f32x4 v;
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] = acc[mi][ni][4 * q + j] * sa;
                        *reinterpret_cast<f32x4*>(prow + c0 + wn * 128 + ni * 32 + cq) = v;
                    }
                }
                continue;
            }
            uint16_t h[4];
            if constexpr (MODE == kGateUp) {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        h[j] = f32_to_bf16_bits(silu(acc[mi][ni][4 * q + j] * sa) * (acc[mi][ni + 2][4 * q + j] * sa));
                    *reinterpret_cast<u32x2*>(out + orow * g.ldo + c0 + wn * 64 + ni * 32 + cq) =
                        u32x2{h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16)};
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) h[j] = f32_to_bf16_bits(acc[mi][ni][4 * q + j] * sa);
                    *reinterpret_cast<u32x2*>(out + orow * g.ldo + c0 + wn * 128 + ni * 32 + cq) =
                        u32x2{h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16)};
                }
            }
        }
    }
}

}  // namespace beam
