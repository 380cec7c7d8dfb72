// FP32 grouped expert GEMMs (layers whose weights and activations are FP32).
//
// One thread per output element with a plain FP32 fma loop: the FP32 path exists for
// small layers where correctness matters and the work is launch-bound, so it is kept
// as simple as possible.  SwiGLU expert (Reflection Beam 1.0 overview, "Mixture of
// Experts"): gate/up rows of w13, SiLU(gate) * up in FP32, then the down projection.
#include "common.cuh"
#include "kernels.h"

namespace beam {

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_simple(int64_t rows, GroupedGemmArgs g,
                                                       const int32_t* __restrict__ ids) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= rows * g.n_out) return;
    const int64_t r = idx / g.n_out;
    const int n = static_cast<int>(idx % g.n_out);
    const int p = g.pair_of_row[r];
    const int e = ids[p];
    const float* a = static_cast<const float*>(g.a) +
                     (g.gather ? static_cast<int64_t>(p / g.topk) : r) * g.lda;
    const float* w = static_cast<const float*>(g.w);
    if (MODE == kGateUp) {
        const int64_t nw = 2 * static_cast<int64_t>(g.n_out);
        const float* wg = w + (static_cast<int64_t>(e) * nw + n) * g.kd;
        const float* wu = wg + static_cast<int64_t>(g.n_out) * g.kd;
        float gs = 0.0f, us = 0.0f;
        for (int k = 0; k < g.kd; ++k) {
            gs = fmaf(a[k], wg[k], gs);
            us = fmaf(a[k], wu[k], us);
        }
        static_cast<float*>(g.out)[r * g.ldo + n] = silu(gs) * us;
    } else {
        const float* wd = w + (static_cast<int64_t>(e) * g.n_out + n) * g.kd;
        float s = 0.0f;
        for (int k = 0; k < g.kd; ++k) s = fmaf(a[k], wd[k], s);
        static_cast<float*>(g.out)[r * g.ldo + n] = s;
    }
}

void launch_gemm_f32(hipStream_t st, GemmMode mode, const GroupedGemmArgs& g, int64_t rows,
                     const int32_t* ids) {
    const int64_t n = rows * g.n_out;
    const int blocks = static_cast<int>((n + 255) / 256);
    if (blocks == 0) return;
    if (mode == kGateUp) gemm_f32_simple<kGateUp><<<blocks, 256, 0, st>>>(rows, g, ids);
    else gemm_f32_simple<kDown><<<blocks, 256, 0, st>>>(rows, g, ids);
}

}  // namespace beam
