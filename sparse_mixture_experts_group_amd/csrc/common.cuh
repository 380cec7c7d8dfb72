// Shared device helpers of libbeam_moe (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace beam {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// FP32 -> BF16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}

// Exponential for the router's sigmoid: Cody & Waite (1980) range reduction
// x = n ln2 + r with n = rint(x log2 e) and ln2 split into a 24-bit-exact high part
// and a low correction, e^r from its Taylor series through r^7/7! in Horner form with
// fused multiply-adds (coefficients are the FP32 roundings of 1/k!), then 2^n by an
// exact ldexp.  The argument is clamped to [-87, 87] so the result stays normal.
// Every step is a single correctly rounded FP32 operation, so the result is the
// same bit pattern on any IEEE FP32 implementation of these operations.
__device__ __forceinline__ float router_exp(float x) {
    x = fminf(fmaxf(x, -87.0f), 87.0f);
    const float kLog2e = 0x1.715476p+0f;
    const float kLn2Hi = 0x1.62e4p-1f;          // 0.693145751953125
    const float kLn2Lo = 0x1.7f7d1cp-20f;       // ln 2 - kLn2Hi
    const float n = __builtin_rintf(__fmul_rn(x, kLog2e));
    float r = __builtin_fmaf(-n, kLn2Hi, x);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 0x1.a01a02p-13f;                  // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, static_cast<int>(n));
}

// Router score s = 1 / (1 + e^-z) with an IEEE round-to-nearest division.
__device__ __forceinline__ float router_sigmoid(float z) {
    return __fdiv_rn(1.0f, __fadd_rn(1.0f, router_exp(-z)));
}

// SiLU for the SwiGLU epilogue (FP32; tolerance-checked, so the fast exp is used).
__device__ __forceinline__ float silu(float g) {
    return g / (1.0f + __expf(-g));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
    return __ballot(p);
}

// Lowest set lane of a nonzero 64-bit mask.
__device__ __forceinline__ int first_lane(uint64_t m) {
    return __builtin_ctzll(m);
}

// A positive normal FP32 block scale s = 2^(c - 127) * m: c, its exponent field, is the
// E8M0 code the scaled MFMAs apply to an operand, and m in [1, 2) its significand, which
// they cannot apply.
__device__ __forceinline__ int scale_e8m0(float s) { return (__float_as_uint(s) >> 23) & 0xff; }
__device__ __forceinline__ float scale_mantissa(float s) {
    return __uint_as_float((__float_as_uint(s) & 0x007fffffu) | 0x3f800000u);
}

// FP32 -> OCP E4M3FN byte, round to nearest even, saturating (gfx950 conversion).
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Block -> (row tile, column tile) map of the prefill grouped GEMMs.
// Workgroups are handed to the 8 XCDs round-robin (hardware id i runs on XCD i % 8), and
// each XCD has its own L2.  Logical block ids are dealt to XCDs in chunks of 32 (one
// block per CU of an XCD), chunk c going to XCD c % 8, so the blocks one XCD runs at a
// time are 32 consecutive logical ids.  Logical ids walk groups of `group_m` row tiles
// across all column tiles, column-major inside a group: 32 consecutive ids cover
// group_m row tiles x 32/group_m column tiles, so activation tiles and weight panels
// are both shared inside an XCD.  The grid covers whole groups in whole chunks of 256.
__device__ __forceinline__ void prefill_tile_of_block(int n_tiles_n, int group_m, int& tile, int& nt) {
    const int i = blockIdx.x;
    const int xcd = i & 7, k = i >> 3;
    const int L = (((k >> 5) << 3) + xcd) * 32 + (k & 31);
    const int per_group = group_m * n_tiles_n;
    const int group = L / per_group, rem = L - group * per_group;
    tile = group * group_m + rem % group_m;
    nt = rem / group_m;
}

// ---------------------------------------------------------------------------
// LDS stages of the prefill GEMMs: each operand row holds 64 bytes of K (32 BF16 or 64
// FP8 values) per stage, filled straight from global memory by global_load_lds_dwordx4.
// One wave instruction writes 1 KB: lane i lands at destination + 16 i, i.e. 16 rows x
// 4 chunks of 16 B.  Chunk c of row r is stored in slot c ^ ((r >> 2) & 3): the 16 rows
// one fragment read serves per LDS cycle (same chunk) then cover all 64 banks.
// ---------------------------------------------------------------------------
constexpr int kStageRowBytes = 64;

__device__ __forceinline__ int stage_offset(int row, int chunk) {
    return row * kStageRowBytes + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// Global byte offset, inside a row's 64-byte K slab, of the chunk lane `lane` moves: a
// DMA instruction covers rows base + lane / 4 (base a multiple of 16), slot lane % 4.
__device__ __forceinline__ int dma_chunk_offset(int lane) {
    return ((lane & 3) ^ ((lane >> 4) & 3)) << 4;
}

// One wave-wide 16-byte-per-lane direct global->LDS load: lane i's 16 bytes from `src`
// land at `lds_dst` + 16 i (lds_dst is wave-uniform).  A plain device function, so
// template code calling it never instantiates the builtin in the host compilation.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}

// A buffer resource over `bytes` bytes from `base` (raw addressing: loads whose offset
// reaches `bytes` return zeros instead of touching memory).  bytes < 2^32.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    // dword 3: a 32-bit data format, as raw dword loads require on gfx9
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(static_cast<uint32_t>(bytes)),
                                             0x00020000);
}

// The buffer form of lds_dma16: lane i's 16 bytes from rsrc base + soff + voff (voff per
// lane, soff wave-uniform) land at lds_dst + 16 i.  32-bit offsets, no per-lane 64-bit
// address arithmetic.
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t rsrc, void* lds_dst, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(lds_dst), 16,
                                             static_cast<int>(voff), soff, 0, 0);
}

// Compile-time loop: f(std::integral_constant<int, i>{}) for i = I .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Scheduling pattern for one K step of NM MFMAs whose next fragments are read before
// its global loads are issued (program order; the compiler keeps LDS reads ahead of
// direct-to-LDS loads it cannot tell apart from them): NR LDS reads spread over the
// first half of the MFMAs, NV loads over the second half, so no MFMA waits behind a
// burst of load issues.
template <int NM, int NR, int NV>
__device__ __forceinline__ void sched_reads_then_loads() {
    constexpr int H1 = NM / 2 > 0 ? NM / 2 : 1, H2 = NM - H1 > 0 ? NM - H1 : 1;
    static_for<0, NM>([](auto i_tag) {
        constexpr int i = decltype(i_tag)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              // MFMA
        if constexpr (i < H1) {
            constexpr int nr = ((i + 1) * NR) / H1 - (i * NR) / H1;
            if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);  // DS read
        } else {
            constexpr int j = i - H1;
            constexpr int nv = ((j + 1) * NV) / H2 - (j * NV) / H2;
            if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);  // VMEM
        }
    });
}

// s_waitcnt vmcnt(N) (expcnt / lgkmcnt left alone): all but the N most recent
// direct-to-LDS loads this wave issued have landed in LDS.  gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15 (no wait).
template <int N>
__device__ __forceinline__ void wait_lds_dma() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for the direct-to-LDS pipelines.  __syncthreads() carries a
// workgroup release fence, which waits for every outstanding vector-memory operation
// (vmcnt(0)) and so would drain the loads of all stages in flight.  Here each wave
// first waits for its own loads of the stage about to be read (wait_lds_dma), then for
// its own LDS reads (so no wave overwrites a stage another wave still reads), then
// meets the others.  The asm statement is also a compiler memory barrier.
__device__ __forceinline__ void lds_pipeline_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // The same wait again as a builtin (a no-op here) so the compiler's wait tracking
    // knows every earlier LDS read has completed and adds no waits for them later.
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Scheduling pattern for one K step of an MFMA loop: NM MFMAs, the first NR of them each
// followed by one LDS read and the next NV each by one global (direct-to-LDS) load, so
// the reads and loads issue while the matrix pipe is busy.  Leftover reads and loads
// follow the last MFMA.
template <int NM, int NR, int NV>
__device__ __forceinline__ void sched_interleave() {
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // DS read
        else if (i < NR + NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
#pragma unroll
    for (int i = NM; i < NR; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = (NM > NR ? NM : NR); i < NR + NV; ++i) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
}

// Calls f(std::integral_constant<int, v>{}) for the wave-uniform v in [0, MI] (MI is 2 or
// 4): a loop body templated on the count of row tiles that hold rows skips the others'
// work with no branch inside the loop.
template <int MI, typename F>
__device__ __forceinline__ void dispatch_row_tiles(int v, F&& f) {
    static_assert(MI == 2 || MI == 4, "row tiles per wave");
    if (v >= MI) {
        f(std::integral_constant<int, MI>{});
    } else if (v <= 0) {
        f(std::integral_constant<int, 0>{});
    } else if constexpr (MI == 4) {
        if (v == 1) f(std::integral_constant<int, 1>{});
        else if (v == 2) f(std::integral_constant<int, 2>{});
        else f(std::integral_constant<int, 3>{});
    } else {
        f(std::integral_constant<int, 1>{});
    }
}

}  // namespace beam
