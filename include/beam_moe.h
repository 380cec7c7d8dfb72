/*
 * beam_moe.h -- C ABI of libbeam_moe.so, the MI355X (gfx950) Beam Mixture-of-Experts layer.
 *
 * The layer (Reflection Beam 1.0 overview, section "Mixture of Experts: 256 experts,
 * 8 routed per token"): a sigmoid router scores E experts (Beam: 256) that form G
 * groups (Beam: 8 groups of 32, contiguous index ranges); the Kg best groups (Beam: 4),
 * ranked by the sum of each group's two largest scores, are kept; the K best experts
 * (Beam: 8) inside the kept groups are picked; each token runs through its K SwiGLU
 * experts (hidden H = 5120, intermediate I = 2560) and the expert outputs are combined
 * with the router scores normalised over the K picks and scaled by alpha = 2.5.  There
 * is no shared expert.  The router, the SwiGLU product and the norms are computed in
 * FP32 (same page, section "Residual stream: depth-dependent weights keep the hidden
 * state at constant scale", last paragraph); GEMMs accumulate in FP32.
 *
 * Conventions for every entry point
 *   - Pointers named "device" point to GPU memory on the current HIP device; the caller
 *     owns every buffer (inputs, outputs, workspace).  The library never allocates or
 *     frees memory and never synchronises the stream.
 *   - All arrays are dense, row-major, 16-byte aligned.  Inputs, outputs and the
 *     workspace must not alias, except h in beam_moe_sublayer_forward (in/out).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call
 *     only enqueues work on it and returns; faults surface at the caller's next sync.
 *   - Arguments are validated on the host before anything is enqueued; on error the
 *     call returns a nonzero beam_status and enqueues nothing.  T == 0 returns BEAM_OK
 *     and enqueues nothing.  No C++ exception crosses this boundary.
 *   - A call that enqueues work first clears the calling thread's last-HIP-error state,
 *     then returns BEAM_ERR_HIP if any of its own launches failed.
 *   - Calls are reentrant; concurrent calls need distinct workspaces.
 *   - Inputs must be finite; non-finite values are not checked for.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *
 * Routing contract (so that the integer result is unique and reproducible):
 *   logits   z[t,e]: the hidden dimension is cut into 64 contiguous chunks of H/64
 *            entries; each chunk is one fused multiply-add chain of x[t,h] * w_router[h,e]
 *            over its h ascending, starting from 0; the 64 chunk sums are added in
 *            ascending chunk order (sum = 0, then sum = sum + chunk_c for c = 0..63),
 *            then + logit_bias[e] (one rounded add) when given.  All FP32, round to
 *            nearest even, no flush of denormals;
 *   scores   s = 1 / (1 + exp(-z)) with exp computed by Cody-Waite reduction and a
 *            degree-7 Taylor polynomial (FP32, argument clamped to [-87, 87]);
 *   order    every ranking is "larger value first, equal values -> lower index first";
 *   weights  w_i = (s_i / d) * alpha, d = s_0 + s_1 + ... + s_{K-1} added in output order.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BEAM_MOE_ABI_VERSION 5

typedef enum {
    BEAM_OK = 0,
    BEAM_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, bad config, misaligned pointer */
    BEAM_ERR_UNSUPPORTED = 2,   /* valid config without kernels (dtype pair, E > 256, ...) */
    BEAM_ERR_WORKSPACE = 3,     /* ws NULL or ws_bytes < beam_moe_workspace_size()       */
    BEAM_ERR_HIP = 4            /* a kernel launch failed (hipGetLastError)               */
} beam_status;

typedef enum {
    BEAM_DTYPE_F32 = 0,
    BEAM_DTYPE_BF16 = 1,
    BEAM_DTYPE_FP8_E4M3 = 2,    /* OCP E4M3FN with one FP32 scale per 128 x 128 block */
    BEAM_DTYPE_MXFP4 = 3        /* OCP MX FP4 (E2M1 elements, E8M0 scale per 32 along K);
                                   weights only */
} beam_dtype;

/*
 * What the caller guarantees about FP8 block scales (beam_moe_config.fp8_scale_kind).
 *   BEAM_FP8_SCALES_FP32  any positive normal FP32 values, e.g. amax / 448 per block
 *                         (the default; every kernel applies the full value)
 *   BEAM_FP8_SCALES_POW2  every scale is a positive power of two (an E8M0 block exponent):
 *                         the LDS-tiled GEMMs then apply only each scale's exponent field,
 *                         through the matrix cores' block scaling, and skip the significand
 *                         fold.  The library does not read the scales on the host to check
 *                         this; with other scales the tiled GEMMs drop their significands.
 * Ignored unless weight_dtype is BEAM_DTYPE_FP8_E4M3.
 */
typedef enum {
    BEAM_FP8_SCALES_FP32 = 0,
    BEAM_FP8_SCALES_POW2 = 1
} beam_fp8_scale_kind;

/*
 * Layer configuration.  Validated on every call:
 *   hidden, inter >= 1; n_experts in [2, 256]; n_groups >= 1 divides n_experts and the
 *   group size S = n_experts / n_groups is >= 2; 1 <= topk_groups <= n_groups;
 *   1 <= topk <= min(32, topk_groups * S); routed_scale finite; fp8_scale_kind is
 *   BEAM_FP8_SCALES_FP32 or BEAM_FP8_SCALES_POW2.
 * Kernel support (else BEAM_ERR_UNSUPPORTED):
 *   (act, weight) in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3), (BF16, MXFP4)};
 *   hidden <= 16384; hidden and inter multiples of 64 for F32 weights; otherwise
 *   hidden a multiple of 256 and inter of 128 (fp8_block must be 128);
 *   with V = ceil(n_experts / 64) scores per lane (V in {1, 2, 4}), S % V == 0 and
 *   S / V a power of two.
 *   Per call, where a GEMM runs LDS-tiled: MXFP4 weights above 256 tokens need
 *   hidden and inter <= 8192; FP8 weights need hidden <= 32768 above 16 tokens and
 *   inter <= 32768 above 103 tokens.
 * Beam: {5120, 2560, 256, 8, 4, 8, 2.5f, BF16, BF16 or FP8_E4M3, 128, 1e-6f, FP32 scales}.
 */
typedef struct beam_moe_config {
    int32_t hidden;        /* H */
    int32_t inter;         /* I, per-expert SwiGLU intermediate size */
    int32_t n_experts;     /* E */
    int32_t n_groups;      /* G */
    int32_t topk_groups;   /* Kg */
    int32_t topk;          /* K */
    float   routed_scale;  /* alpha (2.5) */
    int32_t act_dtype;     /* beam_dtype of x / y (F32 or BF16) */
    int32_t weight_dtype;  /* beam_dtype of w13 / w2 */
    int32_t fp8_block;     /* weight scale block edge for FP8 (128); ignored otherwise */
    float   norm_eps;      /* RMSNorm epsilon (sublayer only) */
    int32_t fp8_scale_kind;  /* beam_fp8_scale_kind (FP8 weights; 0 = general FP32 scales) */
} beam_moe_config;

/* Human-readable name of a beam_status value (static string, never NULL). */
const char* beam_moe_status_string(int status);

/* BEAM_MOE_ABI_VERSION of the built library. */
int beam_moe_abi_version(void);

/*
 * Bytes of device workspace one call with this config and T tokens needs (route,
 * forward and sublayer all fit in it).  Returns 0 for an invalid config or T < 0.
 */
size_t beam_moe_workspace_size(const beam_moe_config* cfg, int64_t T);

/*
 * Router only (Beam overview, "Mixture of Experts": sigmoid scores, group top-2 sums,
 * top-Kg groups, top-K experts, normalised weights x alpha).
 *   x          device [T, H], act_dtype (BF16 values are widened exactly to FP32)
 *   w_router   device [H, E] FP32
 *   logit_bias device [E] FP32 added to each logit before the sigmoid, or NULL
 *   select_bias device [E] FP32 or NULL: a choosing-only expert bias (the balancing
 *              "expert bias" of the Beam training notes, pretraining foundations; the
 *              pages do not say where it enters -- read here as: groups and experts
 *              are ranked by r = s + b, one rounded FP32 add, while the weights
 *              normalise the unbiased scores s of the picks).  NULL: r = s.
 *   ids        device [T, K] int32 out: expert ids, ranking-value-descending, ties ->
 *              lower id
 *   weights    device [T, K] FP32 out: combine weights, summing to alpha per token
 *   ws         device workspace of ws_bytes >= beam_moe_workspace_size(cfg, T)
 */
int beam_moe_route(const beam_moe_config* cfg, int64_t T, const void* x,
                   const float* w_router, const float* logit_bias,
                   const float* select_bias, int32_t* ids, float* weights, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * One MoE layer (Beam overview, "Mixture of Experts"):
 *   y[t] = sum_{i<K} w[t,i] * Wd_e (SiLU(Wg_e x_t) * (Wu_e x_t)),  e = ids[t,i].
 *   x          device [T, H] act_dtype
 *   w_router   device [H, E] FP32;  logit_bias, select_bias device [E] FP32 or NULL
 *              (as in beam_moe_route)
 *   w13        device [E, 2I, H] weight_dtype: rows 0..I-1 gate, rows I..2I-1 up,
 *              each row H-contiguous (MXFP4: [E, 2I, H/2] bytes, element 2j of a
 *              row in the low nibble of byte j, 2j+1 in the high nibble)
 *   w13_scale  FP8: device [E, 2I/128, H/128] FP32 block scales (value = code *
 *              scale of its 128x128 tile), positive normal FP32 values, or powers of
 *              two only when cfg->fp8_scale_kind says so.  MXFP4: device [E, 2I, H/32] uint8 E8M0 codes
 *              (value = E2M1 element * 2^(code - 127) of its block of 32 along K).
 *              NULL for F32 and BF16 weights.
 *   w2         device [E, H, I] weight_dtype (down projection, rows I-contiguous;
 *              MXFP4: [E, H, I/2] bytes)
 *   w2_scale   FP8: device [E, H/128, I/128] FP32 (as w13_scale); MXFP4: [E, H, I/32]
 *              uint8 E8M0; NULL otherwise
 *   y          device [T, H] act_dtype out
 *   ids_out    device [T, K] int32 out, or NULL;  weights_out device [T, K] FP32 or NULL
 * With FP8 or MXFP4 weights the activations entering each GEMM are quantised on the GPU
 * to E4M3 with one FP32 scale per row (the row's amax / 448).
 */
int beam_moe_forward(const beam_moe_config* cfg, int64_t T, const void* x,
                     const float* w_router, const float* logit_bias,
                     const float* select_bias, const void* w13,
                     const void* w13_scale, const void* w2, const void* w2_scale,
                     void* y, int32_t* ids_out, float* weights_out, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Full MoE sublayer with the constant-scale residual (Beam overview, "Residual stream:
 * depth-dependent weights keep the hidden state at constant scale": every sublayer is
 * normalised before and after; at step k the stream keeps sqrt((k-1)/k) of itself and
 * adds 1/sqrt(k) of the sublayer output):
 *   xhat = RMSNorm(h) * pre_gain            (FP32; sum of squares in the fixed order:
 *                                            64 strided fma chains, then a pairwise tree)
 *   y    = MoE(xhat)                         (router on FP32 xhat)
 *   h   <- c1 * h + c2 * RMSNorm(y) * post_gain,  c1 = sqrt((k-1)/k), c2 = 1/sqrt(k)
 *   h          device [T, H] BF16, updated in place (act_dtype must be BF16)
 *   pre_gain, post_gain  device [H] FP32 or NULL (= ones)
 *   step_k     residual step, >= 2
 *   moe_out    device [T, H] BF16 out (y before the post-norm), or NULL
 *   other arguments as in beam_moe_forward.
 */
int beam_moe_sublayer_forward(const beam_moe_config* cfg, int64_t T, void* h,
                              const float* pre_gain, const float* post_gain,
                              int32_t step_k, const float* w_router,
                              const float* logit_bias, const float* select_bias,
                              const void* w13,
                              const void* w13_scale, const void* w2,
                              const void* w2_scale, void* moe_out, int32_t* ids_out,
                              float* weights_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Where the intermediates of the last call live inside a workspace (byte offsets from
 * ws), for inspection by tests and tools.  Regions:
 *   logits       [T, E] FP32 router logits (bias included)
 *   expert_count [E] int32 rows routed to each expert
 *   expert_off   [E+1] int32 exclusive prefix sum of expert_count
 *   row_of_pair  [T*K] int32: row of pair p = t*K + i in the expert-sorted order
 *   pair_of_row  [T*K] int32: inverse permutation (rows of one expert are consecutive,
 *                in ascending pair order)
 *   hidden       [T*K, I] SwiGLU activations in row order (BF16; FP32 for F32 weights)
 *   expert_out   [T*K, H] expert outputs in row order (BF16; FP32 for F32 weights)
 *   scores       [T, E] FP32 sigmoid scores s = 1 / (1 + exp(-z)) of the routing contract
 *   xhat         [T, H] FP32 normalised input RMSNorm(h) * pre_gain (written by the
 *                sublayer call with BF16 activations)
 *   x_q, x_q_scale  FP8 and MXFP4 weights: [T, H] E4M3 codes of the expert input (x, or
 *                xhat in the sublayer call) and [T] FP32 row scales s = amax / 448 (1 for
 *                a zero row): code = E4M3(v * (1/s)), 1/s and the product rounded to FP32
 *   h_q, h_q_scale  the same for the BF16 `hidden` rows: [T*K, I] codes, [T*K] scales
 *                (the dense MLP's calls keep theirs in their own workspace layout)
 *                Other weight types: empty regions.
 * Returns BEAM_OK, or BEAM_ERR_INVALID_ARG for a bad config / T.
 */
typedef struct beam_moe_ws_map {
    size_t logits, expert_count, expert_off, row_of_pair, pair_of_row, hidden, expert_out;
    size_t scores, xhat;
    size_t x_q, x_q_scale, h_q, h_q_scale;
    size_t total;
} beam_moe_ws_map;

int beam_moe_workspace_map(const beam_moe_config* cfg, int64_t T, beam_moe_ws_map* out);

/*
 * Dense SwiGLU MLP (Beam overview, section "Architecture": the first 3 of the 52
 * decoder layers run a dense SwiGLU MLP where the other 49 run the MoE block; the pages
 * do not give its intermediate size):
 *   y[t] = Wd (SiLU(Wg x_t) * (Wu x_t))
 * Of cfg only hidden (H), inter (the dense intermediate size I), act_dtype,
 * weight_dtype, fp8_block, norm_eps and fp8_scale_kind are read (hidden, inter >= 1,
 * dtypes and scale kind in range, norm_eps finite and >= 0, else BEAM_ERR_INVALID_ARG);
 * the router fields are ignored.
 * Kernel support is that of the MoE layer's expert GEMMs (dtype pairs, multiples and
 * per-call limits above), except that the streaming kernels, which read the weights
 * once per 32 rows, serve up to 16 tokens and the LDS-tiled kernels above, and that
 * above 16 tokens MXFP4 weights need hidden <= 8192 and inter a multiple of 512 s, s
 * the least power of two with inter / s <= 8192 (s <= 16).  While the tiles are few
 * both GEMMs split the reduction into slices whose FP32 partial sums the workspace
 * holds.  The weights have the layout of one expert of beam_moe_forward (E = 1):
 *   x          device [T, H] act_dtype
 *   w13        device [2I, H] weight_dtype (rows 0..I-1 gate, I..2I-1 up; MXFP4
 *              [2I, H/2] bytes);  w13_scale FP8 [2I/128, H/128] FP32 (as above),
 *              MXFP4 [2I, H/32] E8M0 codes, NULL otherwise
 *   w2         device [H, I] weight_dtype (MXFP4 [H, I/2]);  w2_scale FP8
 *              [H/128, I/128], MXFP4 [H, I/32], NULL otherwise
 *   y          device [T, H] act_dtype out
 *   ws         device workspace of ws_bytes >= beam_dense_workspace_size(cfg, T)
 * The GEMMs and the E4M3 activation quantisation are those of beam_moe_forward.
 */
size_t beam_dense_workspace_size(const beam_moe_config* cfg, int64_t T);

int beam_dense_forward(const beam_moe_config* cfg, int64_t T, const void* x, const void* w13,
                       const void* w13_scale, const void* w2, const void* w2_scale, void* y,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Dense MLP sublayer with the constant-scale residual (as beam_moe_sublayer_forward
 * with the dense MLP in place of the MoE block):
 *   h <- c1 * h + c2 * RMSNorm(Dense(RMSNorm(h) * pre_gain)) * post_gain
 *   h          device [T, H] BF16, updated in place (act_dtype must be BF16)
 *   mlp_out    device [T, H] BF16 out (the MLP output before the post-norm), or NULL
 *   other arguments as in beam_moe_sublayer_forward and beam_dense_forward.
 */
int beam_dense_sublayer_forward(const beam_moe_config* cfg, int64_t T, void* h,
                                const float* pre_gain, const float* post_gain, int32_t step_k,
                                const void* w13, const void* w13_scale, const void* w2,
                                const void* w2_scale, void* mlp_out, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Kernel timing hook (instrumentation for benchmarks; not needed for computing).
 * After this call, every launch of the selected kernel by later calls from the same host
 * thread is bracketed by hipEventRecord of the next pair of events on the launch stream:
 * launch i records events[2i] before and events[2i+1] after the kernel, for i < n_pairs;
 * later launches are not bracketed.  `events` holds hipEvent_t handles created by the
 * caller (with timing enabled) and must stay valid until the last bracketed launch has
 * been recorded.  kernel: BEAM_KERNEL_NONE disables the hook.  The hook belongs to the
 * calling host thread: calls from other threads are neither bracketed nor disturbed.
 * Returns BEAM_ERR_INVALID_ARG for an unknown kernel id, n_pairs < 0, or events == NULL
 * with n_pairs > 0.
 */
typedef enum {
    BEAM_KERNEL_NONE = 0,
    BEAM_KERNEL_ROUTER_LOGITS = 1,   /* FP32 router logits */
    BEAM_KERNEL_GATE_UP = 2,         /* grouped gate/up GEMM with the SwiGLU epilogue */
    BEAM_KERNEL_DOWN = 3,            /* grouped down-projection GEMM */
    BEAM_KERNEL_COMBINE = 4          /* weighted combine (or combine + post-norm + residual) */
} beam_kernel_id;

int beam_moe_time_kernel(int kernel, void* const* events, int n_pairs);

/*
 * beam_moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The intermediates live in a static device array of
 * BEAM_MOE_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on until
 * the process ends; its address is looked up once per device, on the first call with
 * that device current.  The call allocates nothing and frees nothing.
 *   Arguments and results are those of beam_moe_forward (ids_out / weights_out may be
 *   NULL as there).
 *   Returns BEAM_ERR_WORKSPACE, before anything is enqueued, when
 *   beam_moe_workspace_size(cfg, T) exceeds BEAM_MOE_NOALLOC_SCRATCH_BYTES (Beam's BF16
 *   layer: up to about 300 tokens), and BEAM_ERR_HIP if the scratch address cannot be
 *   found on the current device.
 *   Every call on one device shares that device's array and leaves its contents
 *   behind; nothing in it has to start at zero (each call writes every region it later
 *   reads).  Calls that overlap in time on one device -- from several threads or on
 *   several streams without ordering between them -- race on the array.
 */
#define BEAM_MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int beam_moe_forward_noalloc(const beam_moe_config* cfg, int64_t T, const void* x,
                             const float* w_router, const float* logit_bias,
                             const float* select_bias, const void* w13,
                             const void* w13_scale, const void* w2, const void* w2_scale,
                             void* y, int32_t* ids_out, float* weights_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_MOE_H */
