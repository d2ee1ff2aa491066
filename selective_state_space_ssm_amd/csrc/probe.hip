// probe.hip -- measurement kernels for gfx950, built into libssm_probe.so
// with exactly the flags of the scan library (packed fp32 off, contraction
// off).  They calibrate the bounds the scan kernels are priced against:
//  - instruction issue rates of the operations a state-step is made of
//    (v_fma_f32, v_mul_f32, v_exp_f32, a DPP-modified v_add_f32 and
//    v_permlane16_swap), alone, and exp mixed with four FMAs (the ratio of a
//    state-step), which shows whether the two overlap;
//  - the shader clock while those kernels run (s_memtime cycles against the
//    100 MHz s_memrealtime counter);
//  - the bandwidth a plain streaming copy reaches, the practical HBM ceiling
//    next to the 8 TB/s specification.
// Nothing here is part of the scan library's C ABI; bench.py loads this
// library by itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;   // independent dependency chains per lane

enum Kind {
    K_FMA = 0,        // v_fma_f32
    K_MUL = 1,        // v_mul_f32
    K_EXP = 2,        // v_exp_f32 (2^x), neg/abs input modifiers (free)
    K_MIX41 = 3,      // per chain: 1 v_exp_f32 then 4 v_fma_f32
    K_DPP_ADD = 4,    // v_add_f32 with a DPP row_ror:8 source
    K_SWAP16 = 5,     // v_permlane16_swap_b32 (one instruction swaps two VGPRs' rows)
};

__device__ __forceinline__ float dpp_ror8(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));
}

// Every lane runs `iters` rounds over kChains independent chains; the
// result is stored so that nothing is removed.  Cycle counters of lane 0 of
// each workgroup's first wavefront go to clk[4 * block ...].
template <int KIND>
__global__ __launch_bounds__(256) void rate_kernel(float *out, uint64_t *clk, int iters, float m, float c) {
    const int tid = threadIdx.x;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float a[kChains], b[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        a[k] = 0.001f * (float)(tid + k);
        b[k] = 0.5f + 0.001f * (float)k;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) {
            if constexpr (KIND == K_FMA) {
                a[k] = fmaf(a[k], m, c);
            } else if constexpr (KIND == K_MUL) {
                a[k] = a[k] * m;
            } else if constexpr (KIND == K_EXP) {
                a[k] = __builtin_amdgcn_exp2f(-fabsf(a[k]));
            } else if constexpr (KIND == K_MIX41) {
                const float e = __builtin_amdgcn_exp2f(-fabsf(a[k]));
                a[k] = fmaf(a[k], m, e);
                b[k] = fmaf(b[k], m, e);
                a[k] = fmaf(a[k], m, c);
                b[k] = fmaf(b[k], m, c);
            } else if constexpr (KIND == K_DPP_ADD) {
                a[k] = a[k] + dpp_ror8(a[k]);
            } else if constexpr (KIND == K_SWAP16) {
                const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[k]), __float_as_uint(b[k]),
                                                                false, false);
                a[k] = __uint_as_float(r[0]);
                b[k] = __uint_as_float(r[1]);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += a[k] + b[k];
    out[(size_t)blockIdx.x * blockDim.x + tid] = s;
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
        clk[4 * blockIdx.x + 0] = t0;
        clk[4 * blockIdx.x + 1] = t1;
        clk[4 * blockIdx.x + 2] = r0;
        clk[4 * blockIdx.x + 3] = r1;
    }
}

// Plain streaming copy, 16 bytes per lane per access.  A tile is U * 256
// consecutive elements; a workgroup takes tiles in grid stride and each lane
// issues its U loads (256 elements apart) before its U stores.  The last
// index a tile touches is tile * U * 256 + 255 + (U - 1) * 256, inside the
// tile; the elements after the last whole tile are copied one per lane.
__global__ __launch_bounds__(256) void copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst,
                                                   int64_t n4) {
    constexpr int U = 4, T = 256;
    const int64_t ntiles = n4 / (U * T);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * (U * T) + threadIdx.x;
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = src[base + u * T];
#pragma unroll
        for (int u = 0; u < U; ++u) dst[base + u * T] = v[u];
    }
    const int64_t threads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = ntiles * (U * T) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += threads)
        dst[i] = src[i];
}

}  // namespace

extern "C" {

// Launch one rate kernel of `kind` (see Kind) with `blocks` workgroups of 256
// threads on `stream`.  out: blocks*256 floats; clk: 4*blocks uint64 (device).
// Returns a hipError_t value (0 = success); -1 for an unknown kind.
int probe_rate(int kind, int blocks, int iters, float m, float c, float *out, uint64_t *clk, void *stream) {
    if (blocks < 1 || iters < 1 || !out || !clk) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g((unsigned)blocks), b(256);
    switch (kind) {
        case K_FMA: hipLaunchKernelGGL(rate_kernel<K_FMA>, g, b, 0, s, out, clk, iters, m, c); break;
        case K_MUL: hipLaunchKernelGGL(rate_kernel<K_MUL>, g, b, 0, s, out, clk, iters, m, c); break;
        case K_EXP: hipLaunchKernelGGL(rate_kernel<K_EXP>, g, b, 0, s, out, clk, iters, m, c); break;
        case K_MIX41: hipLaunchKernelGGL(rate_kernel<K_MIX41>, g, b, 0, s, out, clk, iters, m, c); break;
        case K_DPP_ADD: hipLaunchKernelGGL(rate_kernel<K_DPP_ADD>, g, b, 0, s, out, clk, iters, m, c); break;
        case K_SWAP16: hipLaunchKernelGGL(rate_kernel<K_SWAP16>, g, b, 0, s, out, clk, iters, m, c); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}

// Copy n4 16-byte elements from src to dst (device, 16-byte aligned, disjoint).
int probe_copy(const void *src, void *dst, int64_t n4, int blocks, void *stream) {
    if (!src || !dst || n4 < 0 || blocks < 1) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const float4 *>(src), static_cast<float4 *>(dst), n4);
    return (int)hipGetLastError();
}

}  // extern "C"
