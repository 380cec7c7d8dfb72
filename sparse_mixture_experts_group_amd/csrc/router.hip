// Router and token permutation kernels of libbeam_moe.
//
// Router (Reflection Beam 1.0 overview, section "Mixture of Experts: 256 experts,
// 8 routed per token"): sigmoid scores of all experts, groups of E/G contiguous experts
// ranked by the sum of their two largest scores, top-Kg groups kept, top-K experts
// picked inside them, weights = scores normalised over the K picks times alpha.  The
// router runs in FP32 (same page, section "Residual stream ...", last paragraph).
//
// Bit-reproducibility: each logit follows one fixed summation order -- the hidden range
// split into 64 contiguous chunks, each an ascending fused multiply-add chain from 0,
// the chunk sums added in ascending chunk order, then the bias -- the sigmoid uses
// router_exp and IEEE-rounded division, and every ranking is (value desc, index asc),
// so expert ids are a pure function of the input bits.  Contraction is disabled in
// this file so that no a*b+c is fused behind our back.
#pragma clang fp contract(off)

#include "common.cuh"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// logits z[t,e] = fma-chain_h x[t,h] * wr[h,e] (+ bias[e])
// ---------------------------------------------------------------------------
template <bool XBF16>
__device__ __forceinline__ float load_act(const void* x, int64_t i) {
    if constexpr (XBF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(x)[i]);
    else return static_cast<const float*>(x)[i];
}

// Small T: one block per (64 experts, 4 chunks, 16 tokens); wave w of the block owns
// chunk c and lane l expert e, and runs the chunk's fma chain for up to 16 tokens at
// once.  The block first stages its tokens' slice of x (4 chunks wide) in LDS as FP32,
// then each lane streams its expert's weights in batches of 16 hidden entries, the next
// batch in flight while the current one is consumed.  The 64 chunk sums go to `part`
// [64, T, E] and router_logits_reduce adds them in order.
template <bool XBF16>
__global__ __launch_bounds__(256) void router_logits_partial(int T, int H, int E, const void* x,
                                                             const float* __restrict__ wr,
                                                             float* __restrict__ part) {
    extern __shared__ float xs[];             // [16][4 * ch]
    const int ch = H / 64;
    const int hw = 4 * ch;
    const int c0 = blockIdx.y * 4;
    const int t0 = blockIdx.z * 16;
    const int nt = min(16, T - t0);
    // stage x[t0 .. t0+16) x [c0*ch, (c0+4)*ch) as FP32, 4 entries per thread per step
    // (hw is a multiple of 4); within a batch all loads of a thread are issued before
    // its LDS stores
    constexpr int kSteps = 8;
    for (int base = 0; base < 16 * hw; base += 256 * 4 * kSteps) {
        float4 v[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int i = base + (threadIdx.x + s * 256) * 4;
            v[s] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (i < 16 * hw) {
                const int tt = i / hw, hh = i - tt * hw;
                if (tt < nt) {
                    const int64_t src = static_cast<int64_t>(t0 + tt) * H + c0 * ch + hh;
                    v[s] = make_float4(load_act<XBF16>(x, src), load_act<XBF16>(x, src + 1),
                                       load_act<XBF16>(x, src + 2), load_act<XBF16>(x, src + 3));
                }
            }
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int i = base + (threadIdx.x + s * 256) * 4;
            if (i < 16 * hw) *reinterpret_cast<float4*>(&xs[i]) = v[s];
        }
    }
    __syncthreads();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = c0 + w;
    const int e = blockIdx.x * 64 + (threadIdx.x & 63);
    if (e >= E) return;
    const float* xw = xs + w * ch;
    const float* wcol = wr + static_cast<int64_t>(c) * ch * E + e;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    float wv[16], wn[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) wv[u] = u < ch ? wcol[static_cast<int64_t>(u) * E] : 0.0f;
    for (int j0 = 0; j0 < ch; j0 += 16) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
            wn[u] = (j0 + 16 + u < ch) ? wcol[static_cast<int64_t>(j0 + 16 + u) * E] : 0.0f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (j0 + u < ch) {
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = __builtin_fmaf(xw[i * hw + j0 + u], wv[u], acc[i]);
            }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) wv[u] = wn[u];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (i < nt) part[(static_cast<int64_t>(c) * T + t0 + i) * E + e] = acc[i];
}

// Ordered sum of the 64 chunk sums (then the bias) for every (t, e); spread over the
// whole chip, since a few selection waves would need far too long for these loads.
__global__ __launch_bounds__(256) void router_logits_reduce(int T, int E, const float* __restrict__ part,
                                                            const float* __restrict__ bias, float* __restrict__ z) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t n = static_cast<int64_t>(T) * E;
    if (idx >= n) return;
    float pv[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) pv[c] = part[c * n + idx];
    float tot = 0.0f;
#pragma unroll
    for (int c = 0; c < 64; ++c) tot = __fadd_rn(tot, pv[c]);
    if (bias) tot = __fadd_rn(tot, bias[idx % E]);
    z[idx] = tot;
}

// Large T: register-tiled kernel.  Block = BT tokens x BE experts, 256 threads as
// 16 x 16; each thread owns a (BT/16) x (BE/16) tile of outputs with two registers per
// output: the running fma chain of the current chunk and the ordered sum of finished
// chunks.  Tiles of HK hidden entries, HK dividing the chunk length H / 64, are staged
// through LDS (x transposed so a thread's tokens are contiguous), so a chunk ends only
// at a tile end and the fold is one uniform branch per tile.  The global loads of tile
// h0 + HK are issued before the fmas of tile h0 (register double buffering).
template <bool XBF16, int BT, int BE, int HK>
__global__ __launch_bounds__(256) void router_logits_tiled(int T, int H, int E, const void* x,
                                                           const float* __restrict__ wr,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ z) {
    constexpr int TM = BT / 16, TN = BE / 16;
    constexpr int XP = BT + 4;               // padded LDS pitch of the transposed x tile
    __shared__ float xs[HK * XP];
    __shared__ float ws[HK * BE];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
    const int ch = H / 64;

    float acc[TM][TN], tot[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) { acc[i][j] = 0.0f; tot[i][j] = 0.0f; }

    // x tile: BT rows x HK cols, XE consecutive hidden entries per thread; w tile: HK rows
    // x BE cols, WV float4 chunks per thread
    constexpr int XE = (BT * HK + 255) / 256;
    constexpr int XT = HK / XE;              // threads per x row
    static_assert(HK % XE == 0 && BT * XT <= 256, "x tile mapping");
    const int xr = tid / XT, xc = (tid % XT) * XE;
    const bool xon = xr < BT;
    const int xt = min(t0 + min(xr, BT - 1), T - 1);
    constexpr int WV = (HK * BE / 4 + 255) / 256;
    float xv[XE];
    f32x4 wv[WV];          // native vectors: kept in registers
    int64_t xoff = static_cast<int64_t>(xt) * H + xc;
    const float* wp = wr + e0;
    auto w_ok = [&](int i) { return (HK * BE / 4) % 256 == 0 || tid + i * 256 < HK * BE / 4; };
#pragma unroll
    for (int i = 0; i < XE; ++i) xv[i] = load_act<XBF16>(x, xoff + i);
#pragma unroll
    for (int i = 0; i < WV; ++i) {
        const int c = tid + i * 256;
        if (w_ok(i)) wv[i] = *reinterpret_cast<const f32x4*>(wp + static_cast<int64_t>(c / (BE / 4)) * E + (c % (BE / 4)) * 4);
    }
    for (int h0 = 0; h0 < H; h0 += HK) {
        __syncthreads();
        if (xon) {
#pragma unroll
            for (int i = 0; i < XE; ++i) xs[(xc + i) * XP + xr] = xv[i];
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int c = tid + i * 256;
            if (w_ok(i)) *reinterpret_cast<f32x4*>(&ws[(c / (BE / 4)) * BE + (c % (BE / 4)) * 4]) = wv[i];
        }
        __syncthreads();
        if (h0 + HK < H) {
            xoff += HK;
            wp += static_cast<int64_t>(HK) * E;
#pragma unroll
            for (int i = 0; i < XE; ++i) xv[i] = load_act<XBF16>(x, xoff + i);
#pragma unroll
            for (int i = 0; i < WV; ++i) {
                const int c = tid + i * 256;
                if (w_ok(i))
                    wv[i] = *reinterpret_cast<const f32x4*>(wp + static_cast<int64_t>(c / (BE / 4)) * E + (c % (BE / 4)) * 4);
            }
        }
#pragma unroll 8
        for (int k = 0; k < HK; ++k) {
            float a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = xs[k * XP + ty * TM + i];
#pragma unroll
            for (int j = 0; j < TN; ++j) b[j] = ws[k * BE + tx * TN + j];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if ((h0 + HK) % ch == 0) {                 // chunk finished: fold it into the total
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) { tot[i][j] = __fadd_rn(tot[i][j], acc[i][j]); acc[i][j] = 0.0f; }
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int t = t0 + ty * TM + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int e = e0 + tx * TN + j;
            float v = tot[i][j];
            if (bias) v = __fadd_rn(v, bias[e]);
            z[static_cast<int64_t>(t) * E + e] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// selection: one wavefront per token
// ---------------------------------------------------------------------------
// Lane l holds the V scores of experts l*V .. l*V+V-1.  A group of S experts spans
// L = S/V lanes (a power of two), so the group's top-2 pair is reduced with xor
// shuffles inside aligned lane segments.  Each "pick the best" round is a wave-wide
// max followed by a ballot of the lanes holding it; the lowest such lane holds the
// lowest index with that value (lanes are in index order, and a lane's local best is
// its first maximum).  The block also records, for the stable token -> expert
// permutation, how many of its pairs go to each expert and each pair's rank among the
// block's pairs with the same expert.
// Optional selection bias (the balancing "expert bias" of the Beam training notes,
// pretraining foundations section; how it enters routing is not on the pages -- read
// here as a choosing-only bias): groups and experts are ranked by s + b, the weights
// normalise the unbiased scores s of the picks.
template <int V>
__global__ __launch_bounds__(kSelectTokens * 64) void router_select(int T, int E, int G, int Kg, int K,
                                                     float alpha, const float* __restrict__ z,
                                                     const float* __restrict__ sel_bias,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ wts,
                                                     int32_t* __restrict__ blk_cnt,
                                                     int32_t* __restrict__ pair_rank,
                                                     float* __restrict__ scores) {
    __shared__ int32_t s_ids[kSelectTokens * kMaxTopK];
    __shared__ int32_t s_cnt[kMaxExperts];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kSelectTokens;
    for (int i = threadIdx.x; i < E; i += kSelectTokens * 64) s_cnt[i] = 0;

    const int S = E / G;
    const int L = S / V;
    const int group = (lane * V) / S;
    const bool lane_live = lane * V < E;

    {
        const int tl = wave;
        const int t = t0 + tl;
        if (t >= T) goto done;
        // s: scores (they weight the picks); rk: ranking values, s + b with a selection
        // bias (one rounded add), else s
        float s[V], rk[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int e = lane * V + v;
            s[v] = (e < E) ? router_sigmoid(z[static_cast<int64_t>(t) * E + e]) : -INFINITY;
            rk[v] = (e < E && sel_bias) ? __fadd_rn(s[v], sel_bias[e]) : s[v];
        }
        // the scores [T, E] for inspection (the lane's V consecutive experts)
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (lane * V + v < E) scores[static_cast<int64_t>(t) * E + lane * V + v] = s[v];
        // group top-2 of the ranking values (multiset: a repeated maximum counts twice)
        float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            if (lane * V + v >= E) continue;
            if (rk[v] > a1) { a2 = a1; a1 = rk[v]; }
            else if (rk[v] > a2) a2 = rk[v];
        }
        for (int o = 1; o < L; o <<= 1) {
            const float b1 = __shfl_xor(a1, o, kWave), b2 = __shfl_xor(a2, o, kWave);
            const float n1 = fmaxf(a1, b1);
            const float n2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
            a1 = n1; a2 = n2;
        }
        const bool leader = lane_live && (lane % L == 0);
        float gv = leader ? __fadd_rn(a1, a2) : -INFINITY;

        // keep Kg groups
        uint64_t kept = 0;
        for (int r = 0; r < Kg; ++r) {
            const float m = wave_max(gv);
            const int wl = first_lane(wave_ballot(leader && gv == m));
            kept |= 1ull << ((wl * V) / S);
            if (lane == wl) gv = -INFINITY;
        }
        // candidates: experts inside kept groups only (-inf marks the others and the
        // picks already taken; ranking values may be negative with a bias)
        const bool gk = lane_live && ((kept >> group) & 1ull);
        float c[V];
#pragma unroll
        for (int v = 0; v < V; ++v) c[v] = (gk && lane * V + v < E) ? rk[v] : -INFINITY;

        int my_id = 0;
        float my_s = 0.0f;
        for (int i = 0; i < K; ++i) {
            float lb = c[0], ls = s[0];
            int lv = 0;
#pragma unroll
            for (int v = 1; v < V; ++v)
                if (c[v] > lb) { lb = c[v]; ls = s[v]; lv = v; }
            const float m = wave_max(lb);
            const int wl = first_lane(wave_ballot(lb == m));
            const int wv = __shfl(lv, wl, kWave);
            const float ps = __shfl(ls, wl, kWave);      // the pick's unbiased score
            if (lane == wl) {
#pragma unroll
                for (int v = 0; v < V; ++v)
                    if (v == lv) c[v] = -INFINITY;
            }
            if (lane == i) { my_id = wl * V + wv; my_s = ps; }
        }
        float d = 0.0f;
        for (int i = 0; i < K; ++i) d = __fadd_rn(d, __shfl(my_s, i, kWave));
        if (lane < K) {
            const int64_t p = static_cast<int64_t>(t) * K + lane;
            ids[p] = my_id;
            wts[p] = __fmul_rn(__fdiv_rn(my_s, d), alpha);
            s_ids[tl * K + lane] = my_id;
        }
    }
done:
    __syncthreads();
    const int ntok = min(kSelectTokens, T - t0);
    const int np = ntok * K;
    for (int p = threadIdx.x; p < np; p += kSelectTokens * 64) {
        const int e = s_ids[p];
        int r = 0;
        for (int q = 0; q < p; ++q) r += (s_ids[q] == e);
        pair_rank[static_cast<int64_t>(t0) * K + p] = r;
        atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += kSelectTokens * 64) blk_cnt[static_cast<int64_t>(blockIdx.x) * E + i] = s_cnt[i];
}

// ---------------------------------------------------------------------------
// permutation: per-expert counts, offsets, tile list, active-expert list
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int& total) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int add = tid >= o ? sh[tid - o] : 0;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    const int incl = sh[tid];
    total = sh[255];
    __syncthreads();
    return incl - v;
}

// Column scan: block e turns the selection blocks' counts of expert e into exclusive
// per-block offsets within the expert (blk_off) and the expert's total (exp_cnt).
__global__ __launch_bounds__(256) void route_col_scan(int nblk, int E, const int32_t* __restrict__ blk_cnt,
                                                      int32_t* __restrict__ blk_off, int32_t* __restrict__ exp_cnt) {
    __shared__ int sh[256];
    const int e = blockIdx.x;
    int carry = 0;
    for (int b0 = 0; b0 < nblk; b0 += 256) {
        const int b = b0 + threadIdx.x;
        const int v = b < nblk ? blk_cnt[static_cast<int64_t>(b) * E + e] : 0;
        int tot;
        const int ex = block_exclusive_scan(v, sh, tot);
        if (b < nblk) blk_off[static_cast<int64_t>(b) * E + e] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) exp_cnt[e] = carry;
}

// Start of expert e's tiles in the tile list, whose order is: experts by tile count, most
// first (equal counts: lower expert first), each expert's tiles consecutive.  The heavy
// experts' tiles start the grid, so the last blocks to run are light ones; and experts
// with the same count sit together, so when no expert has more than two tiles (a few
// hundred rows per expert) every two-tile expert starts at an even index: its two tiles
// fall in one group of row tiles that an XCD runs side by side (the GEMMs' block order),
// and the second reads each weight panel from that XCD's L2.  s_nt: the tile counts of
// all experts in LDS (written and synchronised by the caller).
__device__ __forceinline__ int tile_list_base(int e, int E, int nt, const int* s_nt) {
    int base = 0;
    for (int i = 0; i < E; ++i) {
        const int n = s_nt[i];
        base += (n > nt || (n == nt && i < e)) ? n : 0;
    }
    return base;
}

// One block of 256 threads; thread e owns expert e (E <= 256): expert offsets, the
// (expert, row-tile) list of the grouped GEMMs and the list of experts with rows.
__global__ __launch_bounds__(256) void route_scan(int E, int BM, const int32_t* __restrict__ exp_cnt,
                                                  int32_t* __restrict__ exp_off, int2* __restrict__ tiles,
                                                  int32_t* __restrict__ meta, int32_t* __restrict__ active) {
    __shared__ int sh[256];
    const int e = threadIdx.x;
    const int tot = e < E ? exp_cnt[e] : 0;
    int total_rows;
    const int base = block_exclusive_scan(tot, sh, total_rows);
    if (e < E) exp_off[e] = base;
    if (e == 0) exp_off[E] = total_rows;
    const int nt = (e < E) ? expert_tile_count(tot, BM) : 0;
    __shared__ int s_nt[kMaxExperts];
    if (e < E) s_nt[e] = nt;
    int total_tiles;
    block_exclusive_scan(nt, sh, total_tiles);       // (its barriers also publish s_nt)
    const int tbase = tile_list_base(e, E, nt, s_nt);
    for (int j = 0; j < nt; ++j) tiles[tbase + j] = make_int2(e, j);
    int n_active;
    const int abase = block_exclusive_scan((e < E && tot > 0) ? 1 : 0, sh, n_active);
    if (e < E && tot > 0) active[abase] = e;
    if (e == 0) {
        meta[kMetaTiles] = total_tiles;
        meta[kMetaActive] = n_active;
    }
}

// Small batches (at most kFinishSmallBlocks selection blocks): one block does the
// column scan, the expert scan / tile list / active list and the scatter, in that order,
// with block barriers in between (saves two launches).
__global__ __launch_bounds__(256) void route_finish_small(int T, int K, int E, int nblk, int BM,
                                                          const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ pair_rank,
                                                          const int32_t* __restrict__ blk_cnt,
                                                          int32_t* __restrict__ blk_off,
                                                          int32_t* __restrict__ exp_cnt,
                                                          int32_t* __restrict__ exp_off, int2* __restrict__ tiles,
                                                          int32_t* __restrict__ meta, int32_t* __restrict__ active,
                                                          int32_t* __restrict__ row_of_pair,
                                                          int32_t* __restrict__ pair_of_row) {
    __shared__ int sh[256];
    __shared__ int s_off[kMaxExperts];
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E) {
        for (int b = 0; b < nblk; ++b) {
            const int64_t i = static_cast<int64_t>(b) * E + e;
            blk_off[i] = tot;
            tot += blk_cnt[i];
        }
        exp_cnt[e] = tot;
    }
    int total_rows;
    const int base = block_exclusive_scan(tot, sh, total_rows);
    if (e < E) { exp_off[e] = base; s_off[e] = base; }
    if (e == 0) exp_off[E] = total_rows;
    const int nt = (e < E) ? expert_tile_count(tot, BM) : 0;
    __shared__ int s_nt[kMaxExperts];
    if (e < E) s_nt[e] = nt;
    int total_tiles;
    block_exclusive_scan(nt, sh, total_tiles);       // (its barriers also publish s_nt)
    const int tbase = tile_list_base(e, E, nt, s_nt);
    for (int j = 0; j < nt; ++j) tiles[tbase + j] = make_int2(e, j);
    int n_active;
    const int abase = block_exclusive_scan((e < E && tot > 0) ? 1 : 0, sh, n_active);
    if (e < E && tot > 0) active[abase] = e;
    if (e == 0) {
        meta[kMetaTiles] = total_tiles;
        meta[kMetaActive] = n_active;
    }
    __syncthreads();      // blk_off written by this block is read back below
    const int64_t npairs = static_cast<int64_t>(T) * K;
    for (int64_t p = threadIdx.x; p < npairs; p += 256) {
        const int64_t b = (p / K) / kSelectTokens;
        const int ee = ids[p];
        const int row = s_off[ee] + blk_off[b * E + ee] + pair_rank[p];
        row_of_pair[p] = row;
        pair_of_row[row] = static_cast<int32_t>(p);
    }
}

// pair p = t*K + i -> row = offset of (its select block, its expert) + its rank.
__global__ __launch_bounds__(256) void route_scatter(int64_t npairs, int K, int E,
                                                     const int32_t* __restrict__ ids,
                                                     const int32_t* __restrict__ pair_rank,
                                                     const int32_t* __restrict__ blk_off,
                                                     const int32_t* __restrict__ exp_off,
                                                     int32_t* __restrict__ row_of_pair,
                                                     int32_t* __restrict__ pair_of_row) {
    const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (p >= npairs) return;
    const int64_t t = p / K;
    const int64_t b = t / kSelectTokens;
    const int e = ids[p];
    const int row = exp_off[e] + blk_off[b * E + e] + pair_rank[p];
    row_of_pair[p] = row;
    pair_of_row[row] = static_cast<int32_t>(p);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
void launch_router_logits(hipStream_t st, int T, int H, int E, bool x_bf16, const void* x,
                          const float* wr, const float* bias, float* z, float* part) {
    if (router_uses_partials(T, H, E)) {
        dim3 grid((E + 63) / 64, 16, (T + 15) / 16);
        const size_t lds = sizeof(float) * 16 * 4 * (H / 64);
        if (x_bf16) router_logits_partial<true><<<grid, 256, lds, st>>>(T, H, E, x, wr, part);
        else router_logits_partial<false><<<grid, 256, lds, st>>>(T, H, E, x, wr, part);
        const int64_t n = static_cast<int64_t>(T) * E;
        router_logits_reduce<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(T, E, part, bias, z);
        return;
    }
    // tile depth: 80 (one whole Beam chunk), else 16; both divide the chunk length
    const int ch = H / 64;
    if (T >= 16384) {
        dim3 grid((T + 63) / 64, E / 128);
        if (ch % 80 == 0) {
            if (x_bf16) router_logits_tiled<true, 64, 128, 80><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
            else router_logits_tiled<false, 64, 128, 80><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
        } else {
            if (x_bf16) router_logits_tiled<true, 64, 128, 16><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
            else router_logits_tiled<false, 64, 128, 16><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
        }
    } else {
        // 64 x 64 tiles (4 x 4 per thread): half the LDS reads per fma of 32 x 128 tiles
        // at the same block count
        dim3 grid((T + 63) / 64, E / 64);
        if (ch % 80 == 0) {
            if (x_bf16) router_logits_tiled<true, 64, 64, 80><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
            else router_logits_tiled<false, 64, 64, 80><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
        } else {
            if (x_bf16) router_logits_tiled<true, 64, 64, 16><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
            else router_logits_tiled<false, 64, 64, 16><<<grid, 256, 0, st>>>(T, H, E, x, wr, bias, z);
        }
    }
}

void launch_router_select(hipStream_t st, int T, int E, int G, int Kg, int K, float alpha,
                          const float* z, const float* sel_bias, int32_t* ids, float* wts, int32_t* blk_cnt,
                          int32_t* pair_rank, float* scores) {
    const int nblk = (T + kSelectTokens - 1) / kSelectTokens;
    const int V = scores_per_lane(E);
    const int nt = kSelectTokens * 64;
#define BEAM_SEL(VV) router_select<VV><<<nblk, nt, 0, st>>>(T, E, G, Kg, K, alpha, z, sel_bias, ids, wts, blk_cnt, pair_rank, scores)
    if (V == 1) BEAM_SEL(1);
    else if (V == 2) BEAM_SEL(2);
    else BEAM_SEL(4);
#undef BEAM_SEL
}

void launch_route_scan(hipStream_t st, int nblk, int E, int BM, const int32_t* blk_cnt,
                       int32_t* blk_off, int32_t* exp_cnt, int32_t* exp_off, int2* tiles,
                       int32_t* meta, int32_t* active) {
    route_col_scan<<<E, 256, 0, st>>>(nblk, E, blk_cnt, blk_off, exp_cnt);
    route_scan<<<1, 256, 0, st>>>(E, BM, exp_cnt, exp_off, tiles, meta, active);
}

void launch_route_scatter(hipStream_t st, int64_t npairs, int K, int E, const int32_t* ids,
                          const int32_t* pair_rank, const int32_t* blk_off, const int32_t* exp_off,
                          int32_t* row_of_pair, int32_t* pair_of_row) {
    const int blocks = static_cast<int>((npairs + 255) / 256);
    route_scatter<<<blocks, 256, 0, st>>>(npairs, K, E, ids, pair_rank, blk_off, exp_off, row_of_pair, pair_of_row);
}

void launch_route_finish_small(hipStream_t st, int T, int K, int E, int nblk, int BM, const int32_t* ids,
                               const int32_t* pair_rank, const int32_t* blk_cnt, int32_t* blk_off,
                               int32_t* exp_cnt, int32_t* exp_off, int2* tiles, int32_t* meta, int32_t* active,
                               int32_t* row_of_pair, int32_t* pair_of_row) {
    route_finish_small<<<1, 256, 0, st>>>(T, K, E, nblk, BM, ids, pair_rank, blk_cnt, blk_off, exp_cnt, exp_off,
                                          tiles, meta, active, row_of_pair, pair_of_row);
}

}  // namespace beam
