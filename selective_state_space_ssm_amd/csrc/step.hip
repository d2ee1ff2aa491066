// step.hip -- one token of batched streaming decode for gfx950.
//
// "mamba, live" (section "what is actually running"): one token in, one out,
// constant work per token; the whole memory is the state h plus a
// (W-1)-token conv history per channel.  For every block k, stream s and
// channel d this kernel shifts the history, applies the causal conv + SiLU,
// takes one recurrence step of every state in place, and writes the gated
// output.
//
// The step is bound by memory traffic on the state (4 B read + 4 B written
// per state coordinate against a handful of VALU ops).  LPC lanes share a
// channel and each holds 4 consecutive states (LPC = 4 up to N = 16), so one
// 16-byte access per lane makes every load and store of the state and of
// A_log one contiguous kilobyte per wavefront (16 channels x 64 B).  The
// per-channel work (conv, softplus, gate) is repeated in the LPC lanes, which
// compute identical values; lane 0 of the channel stores y and the history.
// Every load of a lane is issued before any arithmetic.  The common shape
// (fp32 io, N = 16, a 4-tap conv, D a multiple of 64) runs step_fast_kernel:
// the same arithmetic with unconditional buffer loads on per-row bases.
//
// The state may be stored in bf16 (HT = bf16_t): it is loaded, updated and
// read out in float32 and rounded to bf16 (nearest, ties to even) only when
// stored, which halves the traffic that bounds the step.
//
// With the constant decay source (DISC_CONST: "the s6 cell", section "one
// cell, two architectures") the decay is e^A with no step size, the write is
// B*u and dt_raw is not loaded; the update is the sequence kernel's
// complement form h + (expm1(A) h + B u).
//
// Arithmetic follows the sequence kernel operation by operation: the same
// conv tap order, softplus, decay 2^(dt*A*log2 e) with A = -exp(A_log), and
// the same readout tree -- chains over the sequence kernel's states per
// lane, then its sum over the four lanes of a wavefront, then pairwise
// across its four wavefronts -- so a token-by-token decode reproduces the
// full forward bit for bit.
#include <algorithm>

#include "launch.hpp"
#include "ssm_device.hpp"

namespace ssm {
namespace {

constexpr int kSPL = 4;    // states per lane
enum { DISC_DB = 0, DISC_ZOH = 1, DISC_CONST = 2 };

// LPC lanes per channel, 4 states per lane; VL = states per lane of the
// sequence kernel (its readout chains); MAXW = widest conv carried.
// DTPROJ (the whole-model decode): dt_raw is not loaded but formed as the
// low-rank projection dt_low[s] . dt_w[d] (rank dt_rank), in order of r.
template <typename IOT, typename HT, int LPC, int VL, int DISC, bool CONV, int MAXW, bool DTPROJ = false>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a) {
    const IOT *X = static_cast<const IOT *>(a.x);
    const IOT *DT = static_cast<const IOT *>(a.dt);
    const IOT *Bp = static_cast<const IOT *>(a.Bm);
    const IOT *Cp = static_cast<const IOT *>(a.Cm);
    const IOT *Z = static_cast<const IOT *>(a.z);
    IOT *Y = static_cast<IOT *>(a.y);
    const int64_t D = a.D, N = a.N, S = a.S;
    const int W = a.W;
    // Workgroups walk the (block, stream) rows in order, bpr workgroups of
    // 256 lanes per row of D*LPC lanes.  The row and the lane within it come
    // from 32-bit divisions of workgroup-uniform values (once per wavefront);
    // lanes past the row's end take its last channel's values and store
    // nothing.
    const uint32_t bpr = (uint32_t)((D * LPC + 255) / 256);
    const uint32_t row = blockIdx.x / bpr;                  // k * S + s
    const uint32_t rk = row / (uint32_t)S;
    const int64_t k = rk, s = row - rk * (uint32_t)S;
    const int64_t gl = (int64_t)(blockIdx.x - row * bpr) * 256 + threadIdx.x;
    const bool active = gl < D * LPC;
    const int64_t gc = active ? gl : (D * LPC - 1);
    const int q = (int)(gc & (LPC - 1));
    const int64_t d = gc / LPC;
    const int64_t sd = (k * S + s) * D + d;      // [nblk, S, D]
    const int64_t kd = k * D + d;                // [nblk, D]
    const int n0 = q * kSPL;
    const int nvalid = max(0, min(kSPL, (int)(N - n0)));
    const bool vecN = (N % 4) == 0;

    // ---- loads
    float hq[kSPL], Bq[kSPL], Cq[kSPL], al[kSPL];
    HT *hp = static_cast<HT *>(a.h) + sd * N + n0;
    const int64_t bc = (k * S + s) * N + n0;     // [nblk, S, N]
    load_k_guard<kSPL>(hp, hq, nvalid, vecN);
    load_k_guard<kSPL>(Bp + bc, Bq, nvalid, vecN);
    load_k_guard<kSPL>(Cp + bc, Cq, nvalid, vecN);
    load_k_guard<kSPL>(a.A_log + kd * N + n0, al, nvalid, vecN);
    const float xr = to_f32(X[sd]);
    float dtr = 0.0f;
    if constexpr (DTPROJ) {
        // the channel's LPC lanes take every LPC-th term, then sum over the lanes
        const float *dl = a.dt_low + (k * S + s) * a.dt_rank;
        const float *dw = a.dt_w + kd * a.dt_rank;
        for (int r = q; r < a.dt_rank; r += LPC) dtr = fmaf(dl[r], dw[r], dtr);
        dtr = group_sum<LPC>(dtr);
    } else if constexpr (DISC != DISC_CONST) {
        dtr = to_f32(DT[sd]);
    }
    const float zr = Z != nullptr ? to_f32(Z[sd]) : 0.0f;
    const float dtb = (DISC != DISC_CONST && a.dt_bias) ? a.dt_bias[kd] : 0.0f;
    const float Dd = a.Dskip ? a.Dskip[kd] : 0.0f;
    float hv[MAXW > 1 ? MAXW - 1 : 1], cw[MAXW], cb = 0.0f;
    float *hist = nullptr;
    if constexpr (CONV) {
        if (W > 1) hist = a.conv_state + (k * S + s) * (int64_t)(W - 1) * D + d;   // slot j at hist[j*D]
#pragma unroll
        for (int j = 0; j < MAXW - 1; ++j) hv[j] = (j < W - 1) ? hist[j * D] : 0.0f;
#pragma unroll
        for (int j = 0; j < MAXW; ++j) cw[j] = (j < W) ? a.conv_w[kd * W + j] : 0.0f;
        cb = a.conv_b ? a.conv_b[kd] : 0.0f;
    }

    // ---- arithmetic
    float uu;
    if constexpr (CONV) {
        // bias, then taps oldest to newest
        float acc = cb;
#pragma unroll
        for (int j = 0; j < MAXW - 1; ++j)
            if (j < W - 1) acc = fmaf(cw[j], hv[j], acc);
        float cwl = cw[0];
#pragma unroll
        for (int j = 1; j < MAXW; ++j)
            if (j == W - 1) cwl = cw[j];
        acc = fmaf(cwl, xr, acc);
        uu = silu_f(acc);
    } else {
        uu = xr;
    }
    const float dl = (DISC != DISC_CONST) ? softplus_f(dtr + dtb) : 1.0f;
    const float du = dl * uu;
    float part[kSPL / VL];
#pragma unroll
    for (int gI = 0; gI < kSPL / VL; ++gI) part[gI] = 0.0f;
#pragma unroll
    for (int j = 0; j < kSPL; ++j) {
        const bool v = j < nvalid;
        const float A = neg_exp_f(v ? al[j] : 0.0f);
        const float A2 = v ? A * kLog2e : 0.0f;
        if constexpr (DISC == DISC_CONST) {
            hq[j] += fmaf(expm1f(A), hq[j], uu * Bq[j]);
        } else {
            const float dec = hw_exp2(dl * A2);
            float w;
            if constexpr (DISC == DISC_DB)
                w = du * Bq[j];
            else
                w = expm1f(dl * A) * (1.0f / A) * Bq[j] * uu;
            hq[j] = fmaf(dec, hq[j], w);
        }
        part[j / VL] = fmaf(Cq[j], hq[j], part[j / VL]);
    }
    if (active && nvalid > 0) store_k<kSPL>(hp, hq, nvalid, vecN);
    // the sequence kernel's tree: its chains of VL states, the four chains
    // of a wavefront ((c0 + c3) + (c1 + c2)) at one state per chain with an
    // input-dependent decay, else ((c0 + c1) + (c2 + c3)), then its four
    // wavefronts as ((w0 + w1) + (w2 + w3)); here the lane's four states hold
    // 4/VL chains and the rest of the tree is the pairwise reduction over
    // the channel's LPC lanes
    float ysum;
    if constexpr (VL == 1 && DISC != DISC_CONST)
        ysum = (part[0] + part[3]) + (part[1] + part[2]);
    else if constexpr (VL == 1)
        ysum = (part[0] + part[1]) + (part[2] + part[3]);
    else if constexpr (VL == 2)
        ysum = part[0] + part[1];
    else
        ysum = part[0];
    ysum = group_sum<LPC>(ysum);
    // readout in the sequence kernel's order: (sum_n C h + Dskip*u) * SiLU(z)
    float yv = ysum + Dd * uu;
    if (Z != nullptr) yv *= silu_f(zr);
    if (q == 0 && active) {
        store_io(Y + sd, yv);
        if constexpr (CONV) {
            if (W > 1) {
#pragma unroll
                for (int j = 0; j < MAXW - 2; ++j)
                    if (j < W - 2) hist[j * D] = hv[j + 1];
                hist[(W - 2) * D] = xr;
            }
        }
    }
}

// The common shape on a shorter path: fp32 io, N = 16 (four lanes of four
// states per channel), a 4-tap conv, D a multiple of 64 (every lane of every
// workgroup holds a channel) and below 2^26 (a row's 16 * D state words fit
// 32-bit byte offsets).  The loads are unconditional buffer loads on
// per-row scalar bases with 32-bit lane offsets (no guards, no per-lane 64-bit
// addresses); the arithmetic is step_kernel's for this shape, operation by
// operation, so the two agree bit for bit.
template <typename HT, int DISC>
__global__ __launch_bounds__(256) void step_fast_kernel(StepArgs a) {
    const int64_t D = a.D, S = a.S;
    const uint32_t bpr = (uint32_t)(D / 64);
    const uint32_t row = blockIdx.x / bpr;                  // k * S + s
    const uint32_t rk = row / (uint32_t)S;
    const uint32_t gl = (blockIdx.x - row * bpr) * 256u + threadIdx.x;
    const int q = (int)(gl & 3u);
    const uint32_t d = gl >> 2;
    const int n0 = q * kSPL;
    const float *Xp = static_cast<const float *>(a.x);
    const float *Zp = static_cast<const float *>(a.z);
    float *Yp = static_cast<float *>(a.y);
    HT *Hp = static_cast<HT *>(a.h) + (int64_t)row * D * 16;
    const buf_t rH = make_buf(Hp, (uint64_t)D * 16 * sizeof(HT));
    const buf_t rA = make_buf(a.A_log + (int64_t)rk * D * 16, (uint64_t)D * 64);
    const buf_t rB = make_buf(static_cast<const float *>(a.Bm) + (int64_t)row * 16, 64);
    const buf_t rC = make_buf(static_cast<const float *>(a.Cm) + (int64_t)row * 16, 64);
    const buf_t rX = make_buf(Xp + (int64_t)row * D, (uint64_t)D * 4);
    float *hist = a.conv_state + (int64_t)row * 3 * D;
    const buf_t rHi = make_buf(hist, (uint64_t)D * 12);
    const uint32_t od = d * 4u, oh = (d * 16u + (uint32_t)n0) * (uint32_t)sizeof(HT);

    // ---- loads, all issued before any arithmetic
    float hq[kSPL], Bq[kSPL], Cq[kSPL], al[kSPL], cw[4], hv[3];
    if constexpr (sizeof(HT) == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rH, oh, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) hq[i] = __uint_as_float(v[i]);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rH, oh, 0, 0);
        hq[0] = __uint_as_float(v[0] << 16); hq[1] = __uint_as_float(v[0] & 0xffff0000u);
        hq[2] = __uint_as_float(v[1] << 16); hq[3] = __uint_as_float(v[1] & 0xffff0000u);
    }
    {
        const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rB, (uint32_t)n0 * 4u, 0, 0);
        const auto vc = __builtin_amdgcn_raw_buffer_load_b128(rC, (uint32_t)n0 * 4u, 0, 0);
        const auto va = __builtin_amdgcn_raw_buffer_load_b128(rA, (d * 16u + (uint32_t)n0) * 4u, 0, 0);
        const auto vw = __builtin_amdgcn_raw_buffer_load_b128(make_buf(a.conv_w + (int64_t)rk * D * 4, (uint64_t)D * 16),
                                                             d * 16u, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Bq[i] = __uint_as_float(vb[i]);
            Cq[i] = __uint_as_float(vc[i]);
            al[i] = __uint_as_float(va[i]);
            cw[i] = __uint_as_float(vw[i]);
        }
    }
    const float xr = buf_ld(rX, od, Xp);
    float dtr = 0.0f;
    if constexpr (DISC != DISC_CONST)
        dtr = buf_ld(make_buf(static_cast<const float *>(a.dt) + (int64_t)row * D, (uint64_t)D * 4), od, Xp);
    const float zr = Zp != nullptr ? buf_ld(make_buf(Zp + (int64_t)row * D, (uint64_t)D * 4), od, Xp) : 0.0f;
#pragma unroll
    for (int j = 0; j < 3; ++j) hv[j] = buf_ld(rHi, (uint32_t)j * (uint32_t)D * 4u + od, Xp);
    const int64_t kD = (int64_t)rk * D;
    const float dtb = (DISC != DISC_CONST && a.dt_bias) ? buf_ld(make_buf(a.dt_bias + kD, (uint64_t)D * 4), od, Xp) : 0.0f;
    const float Dd = a.Dskip ? buf_ld(make_buf(a.Dskip + kD, (uint64_t)D * 4), od, Xp) : 0.0f;
    const float cb = a.conv_b ? buf_ld(make_buf(a.conv_b + kD, (uint64_t)D * 4), od, Xp) : 0.0f;

    // ---- arithmetic (step_kernel's, W = 4, four valid states per lane)
    float acc = cb;
#pragma unroll
    for (int j = 0; j < 3; ++j) acc = fmaf(cw[j], hv[j], acc);
    acc = fmaf(cw[3], xr, acc);
    const float uu = silu_f(acc);
    const float dl = (DISC != DISC_CONST) ? softplus_f(dtr + dtb) : 1.0f;
    const float du = dl * uu;
    float part[kSPL];
#pragma unroll
    for (int j = 0; j < kSPL; ++j) part[j] = 0.0f;
#pragma unroll
    for (int j = 0; j < kSPL; ++j) {
        const float A = neg_exp_f(al[j]);
        const float A2 = A * kLog2e;
        if constexpr (DISC == DISC_CONST) {
            hq[j] += fmaf(expm1f(A), hq[j], uu * Bq[j]);
        } else {
            const float dec = hw_exp2(dl * A2);
            float w;
            if constexpr (DISC == DISC_DB)
                w = du * Bq[j];
            else
                w = expm1f(dl * A) * (1.0f / A) * Bq[j] * uu;
            hq[j] = fmaf(dec, hq[j], w);
        }
        part[j] = fmaf(Cq[j], hq[j], part[j]);
    }
    if constexpr (sizeof(HT) == 4) {
        __attribute__((ext_vector_type(4))) unsigned int v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(hq[i]);
        __builtin_amdgcn_raw_buffer_store_b128(v, rH, oh, 0, 0);
    } else {
        __attribute__((ext_vector_type(2))) unsigned int v;
        v[0] = (uint32_t)bf16_rne(hq[0]) | ((uint32_t)bf16_rne(hq[1]) << 16);
        v[1] = (uint32_t)bf16_rne(hq[2]) | ((uint32_t)bf16_rne(hq[3]) << 16);
        __builtin_amdgcn_raw_buffer_store_b64(v, rH, oh, 0, 0);
    }
    float ysum;
    if constexpr (DISC != DISC_CONST)
        ysum = (part[0] + part[3]) + (part[1] + part[2]);
    else
        ysum = (part[0] + part[1]) + (part[2] + part[3]);
    ysum = group_sum<4>(ysum);
    float yv = ysum + Dd * uu;
    if (Zp != nullptr) yv *= silu_f(zr);
    if (q == 0) {
        buf_st(make_buf(Yp + (int64_t)row * D, (uint64_t)D * 4), od, Yp, yv);
        buf_st(rHi, od, hist, hv[1]);
        buf_st(rHi, (uint32_t)D * 4u + od, hist, hv[2]);
        buf_st(rHi, 2u * (uint32_t)D * 4u + od, hist, xr);
    }
}

// One run of workgroups per (block, stream) row: ceil(D*LPC / 256) each.
template <int LPC>
unsigned step_blocks(const StepArgs &a) {
    return (unsigned)(a.nblk * a.S * ((a.D * LPC + 255) / 256));
}

template <typename IOT, typename HT, int LPC, int VL>
hipError_t launch_g(const StepArgs &a, hipStream_t s) {
    const unsigned blocks = step_blocks<LPC>(a);
    const bool conv = a.W > 0;
#define SSM_STEP_CASE(DI, CV, MW)                                                                        \
    if (a.disc == DI && conv == CV && (!CV || a.W <= MW)) {                                              \
        hipLaunchKernelGGL((step_kernel<IOT, HT, LPC, VL, DI, CV, MW>), dim3(blocks), dim3(256), 0, s, a); \
        return hipGetLastError();                                                                        \
    }
    SSM_STEP_CASE(DISC_DB, false, 1)
    SSM_STEP_CASE(DISC_DB, true, 4)
    SSM_STEP_CASE(DISC_DB, true, 8)
    SSM_STEP_CASE(DISC_ZOH, false, 1)
    SSM_STEP_CASE(DISC_ZOH, true, 4)
    SSM_STEP_CASE(DISC_ZOH, true, 8)
    SSM_STEP_CASE(DISC_CONST, false, 1)
    SSM_STEP_CASE(DISC_CONST, true, 4)
    SSM_STEP_CASE(DISC_CONST, true, 8)
#undef SSM_STEP_CASE
    return hipErrorInvalidValue;
}

template <typename IOT, typename HT>
hipError_t launch_io(const StepArgs &a, hipStream_t s) {
    // four states per lane; readout chains = the sequence kernel's states per lane
    if (a.N <= 16) return launch_g<IOT, HT, 4, 1>(a, s);
    if (a.N <= 32) return launch_g<IOT, HT, 8, 2>(a, s);
    return launch_g<IOT, HT, 16, 4>(a, s);
}

}  // namespace

hipError_t launch_step_dtproj(const StepArgs &a, hipStream_t s) {
    if (a.nblk * a.S * a.D == 0) return hipSuccess;
    if (a.bf16 || a.state_bf16 || a.disc != DISC_DB || a.W != 0) return hipErrorInvalidValue;
    if (a.N <= 16)
        hipLaunchKernelGGL((step_kernel<float, float, 4, 1, DISC_DB, false, 1, true>), dim3(step_blocks<4>(a)),
                           dim3(256), 0, s, a);
    else if (a.N <= 32)
        hipLaunchKernelGGL((step_kernel<float, float, 8, 2, DISC_DB, false, 1, true>), dim3(step_blocks<8>(a)),
                           dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((step_kernel<float, float, 16, 4, DISC_DB, false, 1, true>), dim3(step_blocks<16>(a)),
                           dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    if (a.nblk * a.S * a.D == 0) return hipSuccess;
    // the fast path's lane offsets are 32-bit: D * 64 bytes of state per row
    if (!a.bf16 && a.N == 16 && a.W == 4 && a.D % 64 == 0 && a.D < ((int64_t)1 << 26)) {
        const dim3 grid((unsigned)(a.nblk * a.S * (a.D / 64)));
#define SSM_STEP_FAST(DI)                                                                            \
    if (a.disc == DI) {                                                                              \
        if (a.state_bf16)                                                                            \
            hipLaunchKernelGGL((step_fast_kernel<bf16_t, DI>), grid, dim3(256), 0, s, a);            \
        else                                                                                         \
            hipLaunchKernelGGL((step_fast_kernel<float, DI>), grid, dim3(256), 0, s, a);             \
        return hipGetLastError();                                                                    \
    }
        SSM_STEP_FAST(DISC_DB)
        SSM_STEP_FAST(DISC_ZOH)
        SSM_STEP_FAST(DISC_CONST)
#undef SSM_STEP_FAST
    }
    if (a.state_bf16) {
        if (a.bf16) return launch_io<bf16_t, bf16_t>(a, s);
        return launch_io<float, bf16_t>(a, s);
    }
    if (a.bf16) return launch_io<bf16_t, float>(a, s);
    return launch_io<float, float>(a, s);
}

}  // namespace ssm
