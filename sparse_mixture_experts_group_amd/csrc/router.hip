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

typedef float f32x32 __attribute__((ext_vector_type(32)));

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

// Large T on the matrix cores.  The FP32 MFMAs with one K value per instruction
// (v_mfma_f32_32x32x1_2b_f32, v_mfma_f32_16x16x1_4b_f32) add one product per output to
// its accumulator and round once, as an FMA does (checked bit for bit against an exact
// IEEE fma chain on gfx950, denormals included), so a run of them over k is each chunk's
// fma chain in the contract's order, at the FP32 matrix rate (twice the vector FMA rate
// without packed FP32).
// Shapes (lane l, accumulator r):
//   32 x 32 (M16 false): the instruction's two 32 x 32 blocks are the two 32-expert
//     halves of the wave's 64 experts; lane l gives token l % 32's x[t, k] as A and expert
//     l's w[k, e] as B; r holds block r / 16, token 8 ((r % 16) / 4) + 4 (l / 32) + r % 4,
//     expert 32 (r / 16) + l % 32.
//   16 x 16 (M16 true): the four 16 x 16 blocks b are (token half b % 2, expert half
//     b / 2) of 32 tokens x 32 experts (an expert set; WE / 32 sets per wave); lane l gives
//     token l % 32 as A and expert 16 (l / 32) + l % 16 of the set as B; r holds block
//     r / 4, token 4 (l / 16) + r % 4 of its half, expert l % 16 of its half.
// Wave tile: 32 NS tokens x WE experts (the NS token sets share the B values); block: NW
// waves side by side along the experts.  Tiles of 16 hidden entries (a divisor of the
// chunk length H / 64) stream through a ring of S LDS stages filled by direct-to-LDS
// loads, S - 1 tiles ahead: w as [16][WE NW] FP32 (one float per lane and k), x as its
// rows of 16 entries (BF16 or FP32, converted when read; 16-byte pieces of a row placed
// in swizzled slots so the fragment reads of 32 rows spread over the banks).  Every wave
// moves WE / 16 KB of w and 32 NS / NW rows of x per stage, so all waves wait for fixed
// counts.  After each chunk's tiles, each accumulator is added to its running sum (FP32,
// chunk order) and cleared.
template <bool XBF16, int WE, bool M16, int NS, int NW, int S>
__global__ __launch_bounds__(64 * NW) void router_logits_mfma(int T, int H, int E, const void* x,
                                                              const float* __restrict__ wr,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ z) {
    static_assert(WE == 64 || (WE == 32 && M16), "a wave covers 64 experts, or 32 with the 16 x 16 shape");
    constexpr int BT = 32 * NS, BE = WE * NW, HK = 16;
    constexpr int XB = XBF16 ? 2 : 4;                  // bytes per x entry
    constexpr int WSZ = HK * BE * 4, XSZ = BT * HK * XB, STG = WSZ + XSZ;
    constexpr int CPR = XB;                            // 16-byte pieces per x row (16 entries)
    constexpr int XR = BT / NW, XBW = XR * HK * XB;    // x rows and bytes per wave and stage
    constexpr int NXI = (XBW + 1023) / 1024, XL = XBW / NXI / 16;   // its loads, lanes per load
    constexpr int WJ = WE / 16;                        // w loads per wave and stage (1 KB each)
    constexpr int NPS = WJ + NXI;                      // loads per wave and stage
    static_assert(WSZ == NW * WJ * 1024 && (XL == 32 || XL == 64) && NXI * XL * 16 == XBW, "per-wave shares");
    static_assert((S - 2) * NPS < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
    const int rows = min(BT, T - t0);
    const int ntile = H / HK, ch = H / 64;

    // w: instruction j of this wave fills LDS bytes (WJ wave + j) KB of the stage's w
    // area; lane i's 16 bytes are elements q = 256 (WJ wave + j) + 4 i
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wr + e0, static_cast<int64_t>(H) * E * 4 - e0 * 4);
    uint32_t woff[WJ];
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
        const int q = (WJ * wave + j) * 256 + 4 * lane;
        woff[j] = static_cast<uint32_t>((q / BE) * E + q % BE) * 4;
    }
    // x: this wave's rows XR wave .. + XR - 1 (XBW bytes: NXI loads of XL lanes); byte
    // b = 1024 m + 16 i of load m goes to row XR wave + b / (16 XB), slot (b / 16) % CPR,
    // which holds piece slot ^ swizzle(row); rows past T re-read the last token (their
    // sums are not stored)
    auto xswz = [](int r) { return XBF16 ? ((r >> 3) & 1) : ((r >> 2) & 3); };
    const __amdgpu_buffer_rsrc_t rx =
        buffer_rsrc(static_cast<const uint8_t*>(x) + static_cast<int64_t>(t0) * H * XB, static_cast<int64_t>(rows) * H * XB);
    uint32_t xoff[NXI];
#pragma unroll
    for (int m = 0; m < NXI; ++m) {
        const int b = 1024 * m + 16 * lane;
        const int xr = XR * wave + b / (16 * XB), sl = (b / 16) % CPR;
        xoff[m] = static_cast<uint32_t>(min(xr, rows - 1) * H * XB + ((sl ^ xswz(xr)) << 4));
    }
    const bool xlane = lane < XL;

    auto issue = [&](int slot, int tile) {
        uint8_t* st = smem + slot * STG;
#pragma unroll
        for (int j = 0; j < WJ; ++j) lds_dma16_buf(rw, st + (WJ * wave + j) * 1024, woff[j], tile * HK * E * 4);
#pragma unroll
        for (int m = 0; m < NXI; ++m)
            if (XL == 64 || xlane) lds_dma16_buf(rx, st + WSZ + wave * XBW + 1024 * m, xoff[m], tile * HK * XB);
    };

    // accumulator sets: NS token sets x NQ expert sets (32 experts each in the 16 x 16
    // shape, 64 in the 32 x 32 one), RQ values per lane each
    constexpr int NQ = M16 ? WE / 32 : 1, RQ = M16 ? 16 : 32;
    using AccT = std::conditional_t<M16, f32x16, f32x32>;
    AccT acc[NS][NQ], tot[NS][NQ];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int r = 0; r < RQ; ++r) { acc[s][q][r] = 0.0f; tot[s][q][r] = 0.0f; }

#pragma unroll
    for (int i = 0; i < S - 1; ++i) issue(i, min(i, ntile - 1));
    // chunk by chunk (tiles per chunk: ch / 16), the fold after each chunk's tiles, so
    // no branch inside the tile loop splits the accumulators
    const int tpc = ch / HK;
    int n = 0;
    for (int c = 0; c < 64; ++c) {
        for (int u = 0; u < tpc; ++u, ++n) {
            // this wave's loads of tile n have landed once at most the S - 2 later stages
            // (NPS loads each) are in flight; then every wave's have, and no wave still
            // reads the slot refilled below (tile n - 1's)
            wait_lds_dma<(S - 2) * NPS>();
            lds_pipeline_barrier();
            issue((n + S - 1) % S, min(n + S - 1, ntile - 1));
            const uint8_t* st = smem + (n % S) * STG;
            const float* wt = reinterpret_cast<const float*>(st);
            const uint8_t* xt = st + WSZ;
            // every fragment of the tile first (so the reads are in flight together and
            // the MFMAs wait only for the first ones), then the tile's 16 NS MFMAs
            // B: the wave's WE experts, lane l's expert l (32 x 32 shape) or, for expert
            // set q, 32 q + 16 (l / 32) + l % 16 (16 x 16 shape, lanes l and l + 16 alike)
            float a[NS][HK], bv[NQ][HK];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int be = wave * WE + (M16 ? 32 * q + 16 * (lane >> 5) + (lane & 15) : lane);
#pragma unroll
                for (int k = 0; k < HK; ++k) bv[q][k] = wt[k * BE + be];
            }
#pragma unroll
            for (int kk = 0; kk < HK; kk += 4) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int r = 32 * s + (lane & 31);
                    if constexpr (XBF16) {
                        const int pc = (kk >> 3) ^ xswz(r);
                        const u32x2 v = *reinterpret_cast<const u32x2*>(xt + r * 32 + pc * 16 + (kk & 7) * 2);
                        a[s][kk] = __uint_as_float(v[0] << 16);
                        a[s][kk + 1] = __uint_as_float(v[0] & 0xFFFF0000u);
                        a[s][kk + 2] = __uint_as_float(v[1] << 16);
                        a[s][kk + 3] = __uint_as_float(v[1] & 0xFFFF0000u);
                    } else {
                        const int pc = (kk >> 2) ^ xswz(r);
                        const f32x4 v = *reinterpret_cast<const f32x4*>(xt + r * 64 + pc * 16);
#pragma unroll
                        for (int i = 0; i < 4; ++i) a[s][kk + i] = v[i];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);     // keep the reads ahead of the MFMAs
#pragma unroll
            for (int k = 0; k < HK; ++k)
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        if constexpr (M16)
                            acc[s][q] = __builtin_amdgcn_mfma_f32_16x16x1f32(a[s][k], bv[q][k], acc[s][q], 0, 0, 0);
                        else
                            acc[s][q] = __builtin_amdgcn_mfma_f32_32x32x1f32(a[s][k], bv[q][k], acc[s][q], 0, 0, 0);
                    }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int r = 0; r < RQ; ++r) { tot[s][q][r] = __fadd_rn(tot[s][q][r], acc[s][q][r]); acc[s][q][r] = 0.0f; }
    }
    wait_lds_dma<0>();      // the tail's re-loads land before the block's LDS is released
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int r = 0; r < RQ; ++r) {
                // 32 x 32 shape: block r / 16, token 8 ((r % 16) / 4) + 4 (l / 32) + r % 4,
                // expert 32 (r / 16) + l % 32; 16 x 16 shape: block b = r / 4 (token half
                // b % 2, expert half b / 2), token 4 (l / 16) + r % 4, expert l % 16
                const int t = t0 + 32 * s +
                              (M16 ? 16 * ((r >> 2) & 1) + 4 * (lane >> 4) + (r & 3)
                                   : 8 * ((r & 15) >> 2) + 4 * (lane >> 5) + (r & 3));
                const int e = e0 + wave * WE + 32 * q + (M16 ? 16 * (r >> 3) + (lane & 15) : 32 * (r >> 4) + (lane & 31));
                if (t < T) {
                    float v = tot[s][q][r];
                    if (bias) v = __fadd_rn(v, bias[e]);
                    z[static_cast<int64_t>(t) * E + e] = v;
                }
            }
}

template <int WE, bool M16, int NS, int NW, int S>
static void launch_router_mfma(hipStream_t st, bool x_bf16, int T, int H, int E, const void* x, const float* wr,
                               const float* bias, float* z) {
    const dim3 grid((T + 32 * NS - 1) / (32 * NS), E / (WE * NW));
    if (x_bf16) {
        constexpr int lds = S * (16 * WE * NW * 4 + 32 * NS * 16 * 2);
        lds_opt_in(reinterpret_cast<const void*>(&router_logits_mfma<true, WE, M16, NS, NW, S>), lds);
        router_logits_mfma<true, WE, M16, NS, NW, S><<<grid, 64 * NW, lds, st>>>(T, H, E, x, wr, bias, z);
    } else {
        constexpr int lds = S * (16 * WE * NW * 4 + 32 * NS * 16 * 4);
        lds_opt_in(reinterpret_cast<const void*>(&router_logits_mfma<false, WE, M16, NS, NW, S>), lds);
        router_logits_mfma<false, WE, M16, NS, NW, S><<<grid, 64 * NW, lds, st>>>(T, H, E, x, wr, bias, z);
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
// Exclusive prefix sum over the 256 threads of a block (4 waves) in thread order, and the
// total: a shuffle scan inside each wave, the 4 wave totals through LDS (sh[0..3]), two
// barriers (the second so the next call may reuse sh).  Integer sums: exact in any order.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int& total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int t = sh[w];
        before += w < wave ? t : 0;
        tot += t;
    }
    total = tot;
    __syncthreads();
    return before + x - v;
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
// and the second reads each weight panel from that XCD's L2.  s_key: for every one of the
// kMaxExperts slots i, its tile count n_i times 256 plus 255 - i (0 tiles past E), so one
// comparison of keys gives the order; the base is the sum of n_i over the larger keys.
// Every thread reads all keys, four per LDS read, several reads in flight.
static_assert(kMaxExperts == 256, "the scan kernels run one thread per expert slot (256 threads)");
__device__ __forceinline__ int tile_key(int e, int nt) { return nt * 256 + (255 - e); }
__device__ __forceinline__ int tile_list_base(int key, const int* s_key) {
    const int4* v = reinterpret_cast<const int4*>(s_key);
    int base = 0;
#pragma unroll 8
    for (int q = 0; q < kMaxExperts / 4; ++q) {
        const int4 c = v[q];
        base += c.x > key ? c.x >> 8 : 0;
        base += c.y > key ? c.y >> 8 : 0;
        base += c.z > key ? c.z >> 8 : 0;
        base += c.w > key ? c.w >> 8 : 0;
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
    __shared__ __attribute__((aligned(16))) int s_key[kMaxExperts];
    s_key[e] = tile_key(e, nt);                       // 256 threads: every slot, 0 tiles past E
    int total_tiles;
    block_exclusive_scan(nt, sh, total_tiles);       // (its barriers also publish s_key)
    const int tbase = tile_list_base(tile_key(e, nt), s_key);
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
    __shared__ __attribute__((aligned(16))) int s_key[kMaxExperts];
    s_key[e] = tile_key(e, nt);                       // 256 threads: every slot, 0 tiles past E
    int total_tiles;
    block_exclusive_scan(nt, sh, total_tiles);       // (its barriers also publish s_key)
    const int tbase = tile_list_base(tile_key(e, nt), s_key);
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
    // matrix-core kernel (tiles of 16 hidden entries; E a multiple of 128).  Measured on
    // the Beam router (one MI355X): from 16384 tokens, blocks of 64 tokens x 256 experts
    // with 64-expert wave tiles on the 32 x 32 shape (32768 tokens: 0.85 ms, against
    // 1.37 ms for the register-tiled FP32 FMA kernel this replaced); below, 32 tokens x
    // 64 experts with 32-expert wave tiles on the 16 x 16 shape, twice the waves and so
    // two per SIMD at 8192 tokens (4096 tokens BF16: 0.26 against 0.33 ms; 8192 FP32:
    // 0.34 against 0.36; the 64-expert tiles took 0.25 and 0.41)
    if (T >= 16384 && E % 256 == 0) launch_router_mfma<64, false, 2, 4, 4>(st, x_bf16, T, H, E, x, wr, bias, z);
    else launch_router_mfma<32, true, 1, 2, 4>(st, x_bf16, T, H, E, x, wr, bias, z);
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
