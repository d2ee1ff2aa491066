// ssm_device.hpp -- device helpers shared by the gfx950 kernels of the
// selective-scan library: I/O conversion, the per-token elementwise math,
// and in-register wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint16_t bf16_t;

// widest causal conv the kernels carry in registers
#define SSM_MAX_CONV_WIDTH_DEV 8

// ---------------------------------------------------------------- I/O types
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ void store_io(float *p, float v) { *p = v; }
// float -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t bf16_rne(float v) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
    return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void store_io(bf16_t *p, float v) { *p = bf16_rne(v); }

// Load K consecutive io values into floats.  `vec` says the address is
// aligned to the full vector (K*sizeof(T) bytes, capped at 16).
template <int K>
__device__ __forceinline__ void load_k(const float *p, float (&o)[K], bool vec) {
    if constexpr (K % 4 == 0) {
        if (vec) {
#pragma unroll
            for (int i = 0; i < K; i += 4) {
                float4 v = *reinterpret_cast<const float4 *>(p + i);
                o[i] = v.x; o[i + 1] = v.y; o[i + 2] = v.z; o[i + 3] = v.w;
            }
            return;
        }
    } else if constexpr (K == 2) {
        if (vec) {
            float2 v = *reinterpret_cast<const float2 *>(p);
            o[0] = v.x; o[1] = v.y;
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < K; ++i) o[i] = p[i];
}

template <int K>
__device__ __forceinline__ void load_k(const bf16_t *p, float (&o)[K], bool vec) {
    if constexpr (K % 4 == 0) {
        if (vec) {
#pragma unroll
            for (int i = 0; i < K; i += 4) {
                uint2 v = *reinterpret_cast<const uint2 *>(p + i);
                o[i] = __uint_as_float(v.x << 16);
                o[i + 1] = __uint_as_float(v.x & 0xffff0000u);
                o[i + 2] = __uint_as_float(v.y << 16);
                o[i + 3] = __uint_as_float(v.y & 0xffff0000u);
            }
            return;
        }
    } else if constexpr (K == 2) {
        if (vec) {
            uint32_t v = *reinterpret_cast<const uint32_t *>(p);
            o[0] = __uint_as_float(v << 16);
            o[1] = __uint_as_float(v & 0xffff0000u);
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < K; ++i) o[i] = to_f32(p[i]);
}

// Guarded load of K values of which only the first `valid` exist (rest 0).
template <int K, typename T>
__device__ __forceinline__ void load_k_guard(const T *p, float (&o)[K], int valid, bool vec) {
    if (valid >= K) {
        load_k<K>(p, o, vec);
        return;
    }
#pragma unroll
    for (int i = 0; i < K; ++i) o[i] = (i < valid) ? to_f32(p[i]) : 0.0f;
}

template <int K>
__device__ __forceinline__ void store_k(float *p, const float (&v)[K], int valid, bool vec) {
    if constexpr (K % 4 == 0) {
        if (valid >= K && vec) {
#pragma unroll
            for (int i = 0; i < K; i += 4)
                *reinterpret_cast<float4 *>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < K; ++i)
        if (i < valid) p[i] = v[i];
}

// K values rounded to bf16; 8-byte stores of four when `vec` (aligned) and all valid.
template <int K>
__device__ __forceinline__ void store_k(bf16_t *p, const float (&v)[K], int valid, bool vec) {
    if constexpr (K % 4 == 0) {
        if (valid >= K && vec) {
#pragma unroll
            for (int i = 0; i < K; i += 4) {
                const uint32_t lo = (uint32_t)bf16_rne(v[i]) | ((uint32_t)bf16_rne(v[i + 1]) << 16);
                const uint32_t hi = (uint32_t)bf16_rne(v[i + 2]) | ((uint32_t)bf16_rne(v[i + 3]) << 16);
                *reinterpret_cast<uint2 *>(p + i) = make_uint2(lo, hi);
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < K; ++i)
        if (i < valid) p[i] = bf16_rne(v[i]);
}

// ------------------------------------------------------------ buffer access
// Raw buffer descriptors: a uniform 48-bit base, a byte range and the gfx9
// format word (32-bit data).  A lane's byte offset at or past the range
// reads 0 and writes nothing, so tile tails need no per-lane clamping, and
// loads take a 32-bit VGPR offset on a scalar base (no 64-bit address math).
typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr int kBufFormatWord = 0x00020000;

__device__ __forceinline__ buf_t make_buf(const void *base, uint64_t bytes) {
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, kBufFormatWord);
}
__device__ __forceinline__ float buf_ld(buf_t r, uint32_t boff, const float *) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, boff, 0, 0));
}
__device__ __forceinline__ float buf_ld(buf_t r, uint32_t boff, const bf16_t *) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, boff, 0, 0) << 16);
}

// Raw bits of one io value, converted only where the value is used:
// converting right after the load would make the compiler wait for it
// there, ahead of work the load was meant to overlap.
template <typename IOT> struct RawOf { typedef uint32_t type; };
template <> struct RawOf<bf16_t> { typedef uint16_t type; };
__device__ __forceinline__ uint32_t buf_ld_raw(buf_t r, uint32_t boff, const float *) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, boff, 0, 0);
}
__device__ __forceinline__ uint16_t buf_ld_raw(buf_t r, uint32_t boff, const bf16_t *) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, boff, 0, 0);
}
__device__ __forceinline__ float raw_f32(uint32_t v, const float *) { return __uint_as_float(v); }
__device__ __forceinline__ float raw_f32(uint16_t v, const bf16_t *) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ void buf_st(buf_t r, uint32_t boff, float *, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, boff, 0, 0);
}
__device__ __forceinline__ void buf_st(buf_t r, uint32_t boff, bf16_t *, float v) {
    bf16_t h;
    store_io(&h, v);
    __builtin_amdgcn_raw_buffer_store_b16(h, r, boff, 0, 0);
}

// ------------------------------------------------------------ fast math
// Hardware transcendentals (v_exp_f32 = 2^x, v_log_f32 = log2, v_rcp_f32).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(r) = log(1 + e^r) = max(r, 0) + log1p(e^-|r|).  With e in (0, 1]
// and u = fl(1 + e), c = (u - 1) - e is exactly the rounding error of 1 + e
// (u - 1 is exact by Sterbenz's lemma, and so is the difference of two
// numbers within a factor 2 of each other, or c = -e when u == 1), and
// log1p(e) = log(u) - c/(1 + e) + O(c^2).  Dropping the 1/(1 + e) leaves an
// absolute error below |c| e/(1 + e) <= 3e-8, under 1e-7 relative to
// log1p(e); for e below 2^-24, u == 1 and the result is exactly e.  Two
// transcendentals (exp2, log2) instead of a division's third.
__device__ __forceinline__ float softplus_f(float r) {
    const float e = hw_exp2(-fabsf(r) * kLog2e);
    const float u = 1.0f + e;
    const float c = (u - 1.0f) - e;
    return fmaxf(r, 0.0f) + fmaf(hw_log2(u), kLn2, -c);
}

// A = -exp(A_log) through the hardware 2^x (every kernel uses this same
// formula, so the sequence, streaming and backward kernels agree bit for bit
// on the decay; relative error ~3e-7 for |A_log| < 4).
__device__ __forceinline__ float neg_exp_f(float a_log) { return -hw_exp2(a_log * kLog2e); }

// logistic sigmoid and SiLU
__device__ __forceinline__ float sigmoid_f(float x) { return hw_rcp(1.0f + hw_exp2(-x * kLog2e)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (a loop whose
// index is a constant expression, e.g. a DPP lane selector).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------ DPP reductions
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

// Sum over each aligned group of G consecutive lanes (G in 1,2,4,8,16); every
// lane of the group receives the sum.  All 64 lanes must be active.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    if constexpr (G >= 2) v += dpp_f<kDppQuadSwap1>(v);
    if constexpr (G >= 4) v += dpp_f<kDppQuadSwap2>(v);
    if constexpr (G >= 8) v += dpp_f<kDppRowHalfMirror>(v);
    if constexpr (G >= 16) v += dpp_f<kDppRowMirror>(v);
    return v;
}

// Within each 16-lane row, lanes 12..15 receive the sum over lanes
// {p, p-4, p-8, p-12} (the four lanes of the row with the same p mod 4).
// All 64 lanes must be active.
__device__ __forceinline__ float row_stride4_sum(float v) {
    v += dpp_f<kDppRowShr4>(v);
    v += dpp_f<kDppRowShr8>(v);
    return v;
}

// Row (16-lane) operations.  Lane K of the row, broadcast to the whole row.
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
    return dpp_f<0x150 + K>(v);
}

// acc + (lane K of the row's c) * h, as one v_fmac_f32_dpp with a row
// broadcast (the compiler folds a DPP operand into VOP2 multiplies but not
// into the three-operand FMA).  The s_nop gives the two wait states a DPP
// read needs after a VALU write of its source register.
template <int K>
__device__ __forceinline__ float fmac_row_bcast(float acc, float c, float h) {
    asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc) : "v"(c), "v"(h), "n"(K));
    return acc;
}

// Transposed row reduction: p[k] is this lane's partial for token k; lane l
// receives the sum over its 16-lane row of p[l].  Pairings: l^15 (row
// mirror), l^7 (half-row mirror), l^2, l^1; each lane keeps the half of the
// tokens named by its own lane bit, so token bits end equal to lane bits.
//
// The first two pairings split the row at 4-lane bank boundaries (bit 3:
// lanes 0-7 | 8-15; bit 2: lanes 0-3, 8-11 | 4-7, 12-15), so each half is
// one DPP add whose bank mask limits the write to the lanes that keep that
// token (the mask gates only the write, not the lanes the DPP reads from):
// two instructions per pair instead of two selects and an add.  The DPP
// read of a register written by the preceding VALU instruction needs two
// wait states, which the compiler does not see inside asm: each block opens
// with s_nop 1.  All 64 lanes must be active.
__device__ __forceinline__ float row_transpose_sum(const float (&p)[16], int l) {
    float v8[8], v4[4], v2[2];
#define SSM_BANK_PAIR(CTRL, LO, HI, O, X, Y)                                             \
    "v_add_f32_dpp %" #O ", %" #X ", %" #X " " CTRL " row_mask:0xf bank_mask:" LO "\n\t" \
    "v_add_f32_dpp %" #O ", %" #Y ", %" #Y " " CTRL " row_mask:0xf bank_mask:" HI "\n\t"
#pragma unroll
    for (int k = 0; k < 8; k += 2)
        asm("s_nop 1\n\t"
            SSM_BANK_PAIR("row_mirror", "0x3", "0xc", 0, 2, 4)
            SSM_BANK_PAIR("row_mirror", "0x3", "0xc", 1, 3, 5)
            : "=&v"(v8[k]), "=&v"(v8[k + 1])
            : "v"(p[k]), "v"(p[k + 1]), "v"(p[k + 8]), "v"(p[k + 9]));
#pragma unroll
    for (int k = 0; k < 4; k += 2)
        asm("s_nop 1\n\t"
            SSM_BANK_PAIR("row_half_mirror", "0x5", "0xa", 0, 2, 4)
            SSM_BANK_PAIR("row_half_mirror", "0x5", "0xa", 1, 3, 5)
            : "=&v"(v4[k]), "=&v"(v4[k + 1])
            : "v"(v8[k]), "v"(v8[k + 1]), "v"(v8[k + 4]), "v"(v8[k + 5]));
#undef SSM_BANK_PAIR
    const bool b1 = (l & 2) != 0, b0 = (l & 1) != 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float mine = b1 ? v4[k + 2] : v4[k];
        const float send = b1 ? v4[k] : v4[k + 2];
        v2[k] = mine + dpp_f<kDppQuadSwap2>(send);
    }
    const float mine = b0 ? v2[1] : v2[0];
    const float send = b0 ? v2[0] : v2[1];
    return mine + dpp_f<kDppQuadSwap1>(send);
}

// Map a linear block index so that blocks sharing data land on one XCD:
// consecutive logical blocks get consecutive physical slots on the same XCD
// (the hardware deals physical block ids round-robin over `nxcd` XCDs).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks, int nxcd) {
    if (nblocks % nxcd != 0) return bid;
    int64_t per = nblocks / nxcd;
    return (bid % nxcd) * per + bid / nxcd;
}

}  // namespace ssm
