/*
 * CPU oracle for the Beam MoE layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * this code.  The GPU library never calls it and shares no code with it.
 *
 * It holds the FP32 parts of the layer whose result decides an integer (the
 * router: logits, sigmoid, group-limited top-k) and the FP32 pre-norm that feeds
 * the router.  The pages fix these sites to FP32 (Reflection Beam 1.0 overview,
 * section "Residual stream: depth-dependent weights keep the hidden state at
 * constant scale", last paragraph: the router and the norms are computed in FP32).
 * Everything else (expert MLPs, combine, post-norm, residual) is in
 * oracle/__init__.py, in float64 with numpy.
 *
 * Build: gcc -O3 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off -mfma -mavx2
 * (no fast-math; -ffp-contract=off so that every a*b+c not written as fmaf is two
 * roundings, as written).  Denormals are not flushed (x86 default).
 *
 * Fixed operation orders (readings where the pages are silent; both are written out
 * in the design notes): the router dot product is 64 contiguous fused multiply-add
 * chains whose sums are added in order; the pre-norm's sum of squares is 64 strided
 * fused chains followed by a fixed pairwise tree.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* ------------------------------------------------------------------------- */
/* exp and sigmoid                                                            */
/* ------------------------------------------------------------------------- */
/*
 * e^x in FP32 from a published method: Cody & Waite range reduction
 * (W. J. Cody, W. Waite, "Software Manual for the Elementary Functions", 1980):
 *   n = nearest integer to x*log2(e),  r = x - n*ln2  (ln2 split in a high part
 *   with trailing zero bits and a low correction),
 * then e^r by its Taylor series truncated after r^7/7! (|r| <= ln2/2, so the
 * truncation error r^8/8! < 6e-9 relative), evaluated in Horner form, and
 * e^x = 2^n * e^r.  The argument is clamped to [-87, 87], which keeps the result
 * a normal float.
 */
float oracle_expf(float x)
{
    if (x > 87.0f) x = 87.0f;
    if (x < -87.0f) x = -87.0f;
    const float log2e = 1.44269502162933349609375f;      /* FP32(log2 e) */
    const float ln2_hi = 0.693145751953125f;             /* 0x3F317200 */
    const float ln2_lo = 1.428606765330187045e-06f;      /* ln2 - ln2_hi */
    float t = x * log2e;
    float n = rintf(t);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    /* Taylor coefficients 1/k!, each rounded to FP32 */
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* Router score: logistic sigmoid s = 1 / (1 + e^-z), one correctly rounded division.
 * (Reflection Beam 1.0 overview, "Mixture of Experts": every expert is scored with a
 * sigmoid.) */
float oracle_sigmoidf(float z)
{
    return 1.0f / (1.0f + oracle_expf(-z));
}

void oracle_expf_array(int64_t n, const float* x, float* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_expf(x[i]);
}

void oracle_sigmoidf_array(int64_t n, const float* z, float* s)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) s[i] = oracle_sigmoidf(z[i]);
}

/* ------------------------------------------------------------------------- */
/* router logits                                                              */
/* ------------------------------------------------------------------------- */
/*
 * z[t,e] = sum_h x[t,h] * Wr[h,e] (+ bias[e]), FP32.
 * Order contract (the pages fix FP32 for the router but not the summation order):
 * the hidden index range is split into 64 contiguous chunks of H/64 entries; chunk c
 * is one fused multiply-add chain p_c = fma(x[t,h], Wr[h,e], p_c) over its entries in
 * ascending h, starting from 0; the chunk sums are then added in ascending chunk
 * order, z = ((p_0 + p_1) + p_2) + ... + p_63, each a single rounded add (0 + p_0 = p_0
 * exactly); finally z + bias[e], one rounded add.  H must be a multiple of 64.
 * x is FP32 (activations stored in BF16 are widened exactly by the caller).  Wr is
 * [H, E] row-major.  The inner loop runs over e so that every accumulator still sees
 * its own h in ascending order.
 */
void oracle_router_logits(int64_t T, int H, int E, const float* x, const float* wr,
                          const float* bias, float* z)
{
    const int chunk = H / 64;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        float* acc = (float*)malloc(sizeof(float) * (size_t)E);
        float* total = z + t * (int64_t)E;
        for (int e = 0; e < E; ++e) total[e] = 0.0f;
        const float* xr = x + t * (int64_t)H;
        for (int c = 0; c < 64; ++c) {
            for (int e = 0; e < E; ++e) acc[e] = 0.0f;
            for (int h = c * chunk; h < (c + 1) * chunk; ++h) {
                const float xv = xr[h];
                const float* wrow = wr + (int64_t)h * E;
                for (int e = 0; e < E; ++e) acc[e] = fmaf(xv, wrow[e], acc[e]);
            }
            for (int e = 0; e < E; ++e) total[e] = total[e] + acc[e];
        }
        if (bias)
            for (int e = 0; e < E; ++e) total[e] = total[e] + bias[e];
        free(acc);
    }
}

/* ------------------------------------------------------------------------- */
/* group-limited top-k routing                                                */
/* ------------------------------------------------------------------------- */
/*
 * Reflection Beam 1.0 overview, section "Mixture of Experts: 256 experts, 8 routed per
 * token": score all experts with a sigmoid, split them into G groups of E/G
 * (contiguous index ranges), rank the groups by the sum of each group's two largest
 * scores and keep the best Kg, pick the K best experts inside the kept groups, and
 * weight them by their scores normalised over the K picks, times alpha (2.5).  No
 * shared expert.
 *
 * Total order used for every "best" (so the answer is unique): larger value first,
 * equal values -> lower index first.
 * Outputs per token: ids[K] in that order; w[i] = (s_i / d) * alpha with
 * d = ((s_0 + s_1) + s_2) + ... summed in output order.
 * Optional outputs: s_out [T,E] scores, gscore_out [T,G] group scores,
 * gkept_out [T,Kg] kept groups in rank order.
 *
 * Optional selection bias sel_bias [E] (the auxiliary-loss-free balancing bias of the
 * Beam training notes, section on pretraining foundations: "expert bias" updates keep
 * expert load near uniform).  The pages do not say where it enters; the reading taken
 * here: it is added to the scores for choosing only, r_e = s_e + b_e (one rounded FP32
 * add), so groups are ranked by the top-2 sum of r and experts by r, while the weights
 * still normalise the unbiased scores s of the picks.  NULL = no bias (r = s).
 */
void oracle_route(int64_t T, int E, int G, int Kg, int K, float alpha, const float* z,
                  const float* sel_bias, int32_t* ids, float* w, float* s_out,
                  float* gscore_out, int32_t* gkept_out)
{
    const int S = E / G;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        float* s = (float*)malloc(sizeof(float) * (size_t)E);
        float* rk = (float*)malloc(sizeof(float) * (size_t)E);
        float* gs = (float*)malloc(sizeof(float) * (size_t)G);
        char* kept = (char*)calloc((size_t)G, 1);
        char* taken = (char*)calloc((size_t)E, 1);
        for (int e = 0; e < E; ++e) {
            s[e] = oracle_sigmoidf(z[t * (int64_t)E + e]);
            rk[e] = sel_bias ? s[e] + sel_bias[e] : s[e];
        }

        /* group score: top1 + top2 of the ranking values (as a multiset: a repeated
         * maximum counts twice) */
        for (int g = 0; g < G; ++g) {
            float top1 = rk[g * S], top2 = -INFINITY;
            for (int j = 1; j < S; ++j) {
                const float v = rk[g * S + j];
                if (v > top1) { top2 = top1; top1 = v; }
                else if (v > top2) top2 = v;
            }
            gs[g] = top1 + top2;
        }
        /* keep Kg groups */
        for (int r = 0; r < Kg; ++r) {
            int best = -1;
            for (int g = 0; g < G; ++g)
                if (!kept[g] && (best < 0 || gs[g] > gs[best])) best = g;
            kept[best] = 1;
            if (gkept_out) gkept_out[t * Kg + r] = best;
        }
        /* top-K experts among the kept groups' experts only */
        int32_t* out = ids + t * (int64_t)K;
        for (int i = 0; i < K; ++i) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (kept[e / S] && !taken[e] && (best < 0 || rk[e] > rk[best])) best = e;
            taken[best] = 1;
            out[i] = best;
        }
        /* normalised weights, scaled by alpha */
        float d = 0.0f;
        for (int i = 0; i < K; ++i) d = d + s[out[i]];
        for (int i = 0; i < K; ++i) w[t * (int64_t)K + i] = (s[out[i]] / d) * alpha;

        if (s_out)
            for (int e = 0; e < E; ++e) s_out[t * (int64_t)E + e] = s[e];
        if (gscore_out)
            for (int g = 0; g < G; ++g) gscore_out[t * (int64_t)G + g] = gs[g];
        free(s); free(rk); free(gs); free(kept); free(taken);
    }
}

/* ------------------------------------------------------------------------- */
/* pre-norm (RMSNorm) feeding the router                                      */
/* ------------------------------------------------------------------------- */
/*
 * xhat[t,h] = (h[t,h] * r) * gain[h], r = 1 / sqrt(mean_h(h^2) + eps), FP32.
 * (Reflection Beam 1.0 overview, "Residual stream": every sublayer is normalised
 * before and after, norms in FP32; the norm is an RMSNorm.)
 * Order contract for mean(h^2): 64 partial sums, partial l accumulating
 * fma(h, h, .) over the indices h = l, l+64, l+128, ... in ascending order; then
 * the pairwise tree p[l] = p[l] + p[l+o] for o = 32, 16, 8, 4, 2, 1; ms = p[0] / H.
 * gain may be NULL (all ones).
 */
void oracle_prenorm(int64_t T, int H, const float* hin, const float* gain, float eps,
                    float* xhat, float* rstd_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* x = hin + t * (int64_t)H;
        float p[64];
        for (int l = 0; l < 64; ++l) p[l] = 0.0f;
        for (int l = 0; l < 64; ++l)
            for (int h = l; h < H; h += 64) p[l] = fmaf(x[h], x[h], p[l]);
        for (int o = 32; o >= 1; o /= 2)
            for (int l = 0; l < o; ++l) p[l] = p[l] + p[l + o];
        const float ms = p[0] / (float)H;
        const float r = 1.0f / sqrtf(ms + eps);
        float* y = xhat + t * (int64_t)H;
        for (int h = 0; h < H; ++h) y[h] = (x[h] * r) * (gain ? gain[h] : 1.0f);
        if (rstd_out) rstd_out[t] = r;
    }
}

/* OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}
