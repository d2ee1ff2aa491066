// scan_fwd.hip -- forward selective scan for gfx950.
//
// The recurrence (pages: "mamba, live", section "what is actually running";
// "the s6 cell", section "the recurrence"; TensorViz explorer, exact ZOH):
//   dt = softplus(dt_raw + dt_bias),  a = 2^(dt * A * log2 e),  A = -exp(A_log)
//   h  = a * h + coef * B * u,  y = (<h, C> + Dskip * u) * SiLU(z)
//
// Work decomposition.  A block of four wavefronts owns 16 channels of one
// batch row and one time chunk; wavefront w keeps states 4w .. 4w+3 of every
// channel (one state per lane at N = 16), so shapes with B*D/16 = 768 blocks
// put three wavefronts on every SIMD.
// Tokens are processed in tiles of 64:
//  - fetch: the next tile's x, dt_raw, z and its B, C rows are loaded into
//    registers while the current tile is scanned (one tile of prefetch);
//  - stage: the raw conv input goes to LDS (with 8 rows of history for the
//    causal window) and B, C rows go to LDS;
//  - transform: each thread takes one channel and 4 consecutive tokens and
//    computes, once per (token, channel), the conv + SiLU, dt = softplus,
//    dt*u, the gate SiLU(z) and Dskip*u into LDS;
//  - scan: per token a lane reads its channel's (dt, dt*u) and its B, C
//    values from LDS and updates its state with one exp2; the readout
//    <h, C> is summed over a channel's four lanes of the wavefront and
//    across the four wavefronts through LDS.  Inside a wavefront the four
//    lanes are one per 4-lane bank of a row at one state per lane, summed
//    with bank-masked DPP adds as ((0 + 3) + (1 + 2)); at several states per
//    lane they are four 16-lane rows, summed with the gfx950 row swaps
//    v_permlane16/32_swap as ((0 + 1) + (2 + 3)); for the constant decay a
//    lane quad, with DPP, as ((0 + 1) + (2 + 3)).  The wavefronts are summed
//    as ((0 + 1) + (2 + 3)).
// The recurrence itself stays strictly sequential in time inside a chunk.
//
// Decay source ("the s6 cell", section "one cell, two architectures": one
// diagonal cell h = a*h + b*u, two parameterisations).  DISC_DB and DISC_ZOH
// compute the decay from the input at every token (one exp2 per state and
// token).  DISC_CONST fixes it per (channel, state), a = e^A, so it is
// computed once per lane before the time loop; the write is B*u and dt_raw is
// never loaded.  The update is taken in complement form,
// h + ((a - 1) h + w) with a - 1 = expm1(A): a decay close to 1 (a long
// memory) stored as a float32 would carry an error of half an ulp of 1 in
// its distance from 1, which the state amplifies by up to 1/(1 - a); the
// complement keeps that distance to float32's relative precision.  Per
// state and token this is a multiply, two FMAs and an add, no exp.  The time
// split below sees dt = 1 per token.
//
// Long sequences with few independent channels are split in time (two-level
// scan): MODE_LOCAL scans every chunk from a zero state and records its end
// state W_k and sum of dt S_k; carry_kernel walks the chunks in order with
// H_{k+1} = 2^(A*log2e*S_k) * H_k + W_k, the associative composition of the
// chunk's affine maps; MODE_FINAL then re-scans every chunk from its exact
// starting state H_k and writes y.  Time order inside a chunk is untouched.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "launch.hpp"
#include "ssm_device.hpp"

namespace ssm {
namespace {

constexpr int kCPW = 16;            // channels per block
constexpr int kNumXcd = 8;          // XCDs of an MI355X
enum { MODE_FINAL = 0, MODE_LOCAL = 1 };
enum { DISC_DB = 0, DISC_ZOH = 1, DISC_CONST = 2 };

struct FwdParams {
    const void *x, *dt;
    const float *dt_bias, *A_log;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *conv_w, *conv_b;
    const float *conv_hist;        // history for t < 0: [B, W-1, D]
    float *conv_state_out;
    const float *init;             // starting states, nullable
    int64_t init_bstride, init_kstride;
    float *hT;
    void *y;
    float *agg_h;                  // MODE_LOCAL: [B, K, D, N] end states
    float *agg_s;                  // MODE_LOCAL: [B, K, D] sums of dt
    int64_t B, L, D, N;
    int W;
    int64_t chunk;
    int K;                         // chunks along time (array stride)
    int Kgrid;                     // chunks covered by this launch (0 .. Kgrid-1)
    int groups;                    // channel groups of kCPW per batch row
};

constexpr int kTile = 64;           // tokens staged per tile
constexpr int kXS = 20;             // LDS row stride: 16 channels + 4, so the two row groups a
                                    // half-wavefront touches land on disjoint banks
constexpr int kThreads = 256;       // four wavefronts per block
constexpr int kRows = kTile / 16;   // tile rows per thread in the transform role

// Raw loads of one tile, held in registers while the previous tile is
// scanned.  Transform role: thread -> channel tc = tid & 15 and rows
// kRows*rp .. kRows*rp + kRows-1 with rp = tid >> 4.  B and C: the [64][NP]
// element tiles dealt over the block's threads in order, B first then C
// (consecutive threads read consecutive elements).
// The values are kept as raw io bits and converted where they are staged
// or used (for bf16 a conversion right after the load would be a wait).
template <typename IOT, int NP>
struct RawTile {
    static constexpr int TE = kTile * NP;                 // elements per tensor tile
    static_assert(TE % kThreads == 0, "tile elements");
    static constexpr int BCS = 2 * TE / kThreads;
    typedef typename RawOf<IOT>::type raw_t;
    raw_t x[kRows], dt[kRows], z[kRows];
    raw_t bc[BCS];
    __device__ __forceinline__ static float f(raw_t v) { return raw_f32(v, (const IOT *)nullptr); }
};

// Per-thread byte offsets of the fetch inside a tile, the same for every
// tile.  x, dt_raw, z: rows rp*kRows + i of channel tdc; B, C: chunk i of the
// [64][NP] tile, i.e. element ec = (i % per) * kThreads + tid at row ec / NP,
// state ec % NP.
struct FetchOff {
    uint32_t x0, xrow;     // row rp*kRows, and the byte stride of one row
    uint32_t bc0, bcstep;  // chunk 0, and the byte stride between chunks
};

// Loads of one tile through buffer descriptors whose range ends at the end
// of the sequence: rows past L read 0, rows past the tile's end (a chunk
// boundary) are read but never used, states past N are zeroed at staging.
// Every load is unconditional, so the compiler never waits on one (or on
// anything issued before it) until the data is staged.
template <typename IOT, int NP, bool WANT_C, bool WANT_DT>
__device__ __forceinline__ void load_raw(RawTile<IOT, NP> &r, const FetchOff &fo, const IOT *X, const IOT *DT,
                                         const IOT *Z, const IOT *Bp, const IOT *Cp, int64_t b, int64_t L,
                                         int64_t D, int64_t N, int64_t ts) {
    constexpr int TE = RawTile<IOT, NP>::TE;
    constexpr int per = TE / kThreads;                    // loads per tensor per thread
    const uint64_t es = sizeof(IOT);
    const int64_t left = L - ts;                          // tokens from ts to the end
    const buf_t rB = make_buf(Bp + (b * L + ts) * N, (uint64_t)(left * N) * es);
    const buf_t rC = make_buf(Cp + (b * L + ts) * N, (uint64_t)(left * N) * es);
#pragma unroll
    for (int i = 0; i < RawTile<IOT, NP>::BCS; ++i) {
        const int tens = i / per;                         // 0: B, 1: C (compile time)
        const uint32_t off = fo.bc0 + (uint32_t)(i % per) * fo.bcstep;
        r.bc[i] = (tens < (WANT_C ? 2 : 1)) ? buf_ld_raw(tens == 0 ? rB : rC, off, Bp) : 0;
    }
    const uint64_t tb = (uint64_t)(left * D) * es;
    const buf_t rX = make_buf(X + (b * L + ts) * D, tb);
#pragma unroll
    for (int i = 0; i < kRows; ++i) r.x[i] = buf_ld_raw(rX, fo.x0 + (uint32_t)i * fo.xrow, X);
    if constexpr (WANT_DT) {
        const buf_t rD = make_buf(DT + (b * L + ts) * D, tb);
#pragma unroll
        for (int i = 0; i < kRows; ++i) r.dt[i] = buf_ld_raw(rD, fo.x0 + (uint32_t)i * fo.xrow, DT);
    } else {
#pragma unroll
        for (int i = 0; i < kRows; ++i) r.dt[i] = 0;
    }
    if (Z != nullptr) {
        const buf_t rZ = make_buf(Z + (b * L + ts) * D, tb);
#pragma unroll
        for (int i = 0; i < kRows; ++i) r.z[i] = buf_ld_raw(rZ, fo.x0 + (uint32_t)i * fo.xrow, Z);
    } else {
#pragma unroll
        for (int i = 0; i < kRows; ++i) r.z[i] = 0;
    }
}

// B and C go to LDS transposed, [state][token] with a padded row of
// kTile + 4 floats, so that a lane reads four consecutive tokens of its
// state with one 16-byte access.  States past N are staged as zeros.
constexpr int kTS = kTile + 4;

template <typename IOT, int NP, bool WANT_C>
__device__ __forceinline__ void store_bc(const RawTile<IOT, NP> &r, float *sB, float *sC, int tid, int64_t N) {
    constexpr int TE = RawTile<IOT, NP>::TE;
#pragma unroll
    for (int i = 0; i < RawTile<IOT, NP>::BCS; ++i) {
        constexpr int per = TE / kThreads;
        const int tens = i / per;
        const int ec = (i % per) * kThreads + tid;
        const int row = ec / NP, n = ec % NP;
        if (tens < (WANT_C ? 2 : 1)) (tens == 0 ? sB : sC)[n * kTS + row] = (n < N) ? r.f(r.bc[i]) : 0.0f;
    }
}

// Sums over the four 16-lane rows of a wavefront, with the gfx950 row swaps:
// v_permlane16_swap(x, y) returns the rows (x0, y0, x2, y2) and
// (x1, y1, x3, y3), v_permlane32_swap(x, y) the rows (x0, x1, y0, y1) and
// (x2, x3, y2, y3).  Both sums associate as ((row0 + row1) + (row2 + row3)).
__device__ __forceinline__ void swap16(float x, float y, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float y, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// p[i] is this lane's partial for token i; row k receives the sum over the
// four rows of p[k] (for the lane's position in the row).
__device__ __forceinline__ float rows_transpose_sum(const float (&p)[4]) {
    float a0, a1, b0, b1, c0, c1;
    swap16(p[0], p[1], a0, a1);   // rows: p0.r0 p1.r0 p0.r2 p1.r2 | p0.r1 p1.r1 p0.r3 p1.r3
    swap16(p[2], p[3], b0, b1);
    swap32(a0 + a1, b0 + b1, c0, c1);
    return c0 + c1;
}
// Sums over the four 4-lane banks of each 16-lane row, with bank-masked DPP
// adds.  In every row the lanes {c, 7-c, 8+c, 15-c} (c = 0..3) form a group,
// one lane per bank: row_mirror pairs lanes i and 15-i, row_half_mirror
// lanes i and 7-i of each half, and both pairings stay inside a group.
// p[k] is this lane's partial for token k; the lane in bank k receives its
// group's sum for token k, associated as (bank0 + bank3) + (bank1 + bank2).
// The first step leaves tokens 0, 1 in banks 0-1 and tokens 2, 3 in banks
// 2-3, each summed over a mirrored lane pair; the second adds the two pairs.
// All 64 lanes must be active.  A DPP read needs two wait states after the
// VALU write of its source (the s_nop; the compiler does not insert them
// for inline asm).
__device__ __forceinline__ float banks_transpose_sum(const float (&p)[4]) {
    float v0, v1, y;
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %2, %2 row_mirror row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %0, %4, %4 row_mirror row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %1, %3, %3 row_mirror row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %1, %5, %5 row_mirror row_mask:0xf bank_mask:0xc"
        : "=&v"(v0), "=&v"(v1)
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]));
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xa"
        : "=&v"(y)
        : "v"(v0), "v"(v1));
    return y;
}
// Two banks_transpose_sum of four tokens each, interleaved so that no DPP
// read follows the write of its source closer than two instructions.
__device__ __forceinline__ void banks_transpose_sum2(const float (&p)[4], const float (&q)[4], float &yp, float &yq) {
    float a0, a1, b0, b1;
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %6, %6 row_mirror row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %0, %8, %8 row_mirror row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %1, %7, %7 row_mirror row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %1, %9, %9 row_mirror row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %2, %10, %10 row_mirror row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %2, %12, %12 row_mirror row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %3, %11, %11 row_mirror row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %3, %13, %13 row_mirror row_mask:0xf bank_mask:0xc\n\t"
        "v_add_f32_dpp %4, %0, %0 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %4, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
        "v_add_f32_dpp %5, %2, %2 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %5, %3, %3 row_half_mirror row_mask:0xf bank_mask:0xa"
        : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1), "=&v"(yp), "=&v"(yq)
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]));
}
// Every lane of a bank group receives the group's sum, in the same
// association as banks_transpose_sum.
__device__ __forceinline__ float banks_sum(float v) {
    v += dpp_f<kDppRowMirror>(v);
    v += dpp_f<kDppRowHalfMirror>(v);
    return v;
}
// Lane G of each 4-lane bank, broadcast to the bank (DPP quad_perm [G,G,G,G]).
template <int G>
__device__ __forceinline__ float bank_bcast(float v) {
    return dpp_f<G * 0x55>(v);
}
// Quad transpose-reduce: lane j of each lane quad holds partial sums p[i]
// for four consecutive tokens; on return lane j holds the quad's sum for
// token j, associated as ((lane0 + lane1) + (lane2 + lane3)).
__device__ __forceinline__ float quad_transpose_sum(const float (&p)[4], int j) {
    const bool odd = (j & 1) != 0, high = (j & 2) != 0;
    float v[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const float mine = odd ? p[2 * m + 1] : p[2 * m];
        const float send = odd ? p[2 * m] : p[2 * m + 1];
        v[m] = mine + dpp_f<kDppQuadSwap1>(send);
    }
    const float mine = high ? v[1] : v[0];
    const float send = high ? v[0] : v[1];
    return mine + dpp_f<kDppQuadSwap2>(send);
}
// Every row receives the sum over the four rows.
__device__ __forceinline__ float rows_sum(float v) {
    float a, b, c, e;
    swap16(v, v, a, b);
    swap32(a + b, a + b, c, e);
    return c + e;
}

template <int K>
__device__ __forceinline__ void lds_read_k(const float *p, float (&o)[K]) {
    if constexpr (K % 4 == 0) {
#pragma unroll
        for (int i = 0; i < K; i += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(p + i);
            o[i] = v.x; o[i + 1] = v.y; o[i + 2] = v.z; o[i + 3] = v.w;
        }
    } else if constexpr (K == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        o[0] = v.x; o[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < K; ++i) o[i] = p[i];
    }
}

// One block = four wavefronts = 16 channels of one batch row and one time
// chunk.  Wavefront w holds states n = (4w + j)*SPL .. +SPL-1 of each
// channel in the lanes of index j:
//  - one state per lane (N <= 16): j is the lane's 4-lane bank, and channel
//    4r + c of row r sits in lanes c, 7-c, 8+c, 15-c of the row (banks 0..3),
//    the groups that banks_transpose_sum reduces with DPP;
//  - several states per lane: j is the lane's row, channel ch its position
//    in the row, reduced with the gfx950 row swaps.
// The constant decay, whose scan has no exp to hide the reduction's latency
// behind, keeps the four lanes of a channel in a quad instead (lane 4 ch + j)
// and sums them with DPP.
template <typename IOT, int SPL, int DISC, bool CONV, int MODE, int CW = 0>
__global__ __launch_bounds__(kThreads) void scan_fwd_kernel(FwdParams p) {
    constexpr int T = kTile;
    constexpr int NP = 16 * SPL;
    constexpr bool FINAL = MODE == MODE_FINAL;
    // LDS, token-minor ([channel or state][token]) with padded rows
    __shared__ float s_x[CONV ? (T + 8) * kXS : 1];               // raw conv input, [token][channel]
    __shared__ __align__(16) float2 s_dl[kCPW][T + 2];            // {dt, dt*u} (ZOH: {dt, u})
    __shared__ __align__(16) float2 s_gd[FINAL ? kCPW : 1][T + 2];  // {gate, Dskip*u}
    __shared__ __align__(16) float s_B[NP * kTS];
    __shared__ __align__(16) float s_C[FINAL ? NP * kTS : 1];
    __shared__ __align__(16) float s_yp[FINAL ? 4 : 1][FINAL ? kCPW : 1][kTS];  // per-wavefront readout partials

    const IOT *X = static_cast<const IOT *>(p.x);
    const IOT *DT = static_cast<const IOT *>(p.dt);
    const IOT *Bp = static_cast<const IOT *>(p.Bm);
    const IOT *Cp = static_cast<const IOT *>(p.Cm);
    const IOT *Z = FINAL ? static_cast<const IOT *>(p.z) : nullptr;
    IOT *Y = static_cast<IOT *>(p.y);

    const int tid = threadIdx.x;
    // XCD-aware order: the hardware deals block ids round-robin over the 8
    // XCDs; remapping gives each XCD a contiguous range of logical blocks, so
    // neighbouring channel groups (which share 128-byte lines of every token
    // row) and all groups of one batch row (which share its B, C rows) meet
    // in the same L2.
    const int64_t bid = xcd_remap((int64_t)blockIdx.x, (int64_t)gridDim.x, kNumXcd);
    const int64_t g = bid % p.groups;
    const int64_t rest = bid / p.groups;
    const int k = (int)(rest % p.Kgrid);
    const int64_t b = rest / p.Kgrid;
    const int64_t N = p.N, D = p.D, L = p.L;
    const int64_t d0 = g * kCPW;
    const int64_t t0 = (int64_t)k * p.chunk;
    const int64_t t1 = min(L, t0 + p.chunk);
    const int ntiles = (int)((t1 - t0 + T - 1) / T);

    // scan role
    const int wv = tid >> 6, lane = tid & 63;
    constexpr bool kRowsOfStates = DISC != DISC_CONST;
    constexpr bool kBanks = kRowsOfStates && SPL == 1;
    const int bank = (lane >> 2) & 3, q4 = lane & 3;
    const int ch = kBanks ? 4 * (lane >> 4) + ((bank & 1) ? 3 - q4 : q4)
                          : (kRowsOfStates ? (lane & 15) : (lane >> 2));
    const int j = kBanks ? bank : (kRowsOfStates ? (lane >> 4) : (lane & 3));
    const int64_t d = d0 + ch;
    const bool dvalid = d < D;
    const int64_t dc = dvalid ? d : (D - 1);
    const int n0 = (wv * 4 + j) * SPL;
    const int nvalid = max(0, min(SPL, (int)(N - n0)));
    const bool vecN = (N % 4) == 0;
    // transform / output role
    const int tc = tid & 15, rp = tid >> 4;
    const int64_t td = d0 + tc;
    const bool tvalid = td < D;
    const int64_t tdc = tvalid ? td : (D - 1);

    float A2[SPL], An[SPL], Ainv[SPL], h[SPL], am1[DISC == DISC_CONST ? SPL : 1];
#pragma unroll
    for (int s = 0; s < SPL; ++s) h[s] = 0.0f;
    // The starting state is requested first, so the wait for A_log below
    // (issued after it) also covers it; it is then pinned, so that the
    // compiler sees it complete before the loop.  Left pending, it would
    // make the compiler wait for every load in flight at its first use in
    // the loop, on every tile.
    if (p.init != nullptr && nvalid > 0)
        load_k_guard<SPL>(p.init + b * p.init_bstride + (int64_t)k * p.init_kstride + dc * N + n0, h, nvalid,
                          vecN && (SPL % 4 == 0));
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
        const bool v = s < nvalid;
        const float A = neg_exp_f(v ? p.A_log[dc * N + n0 + s] : 0.0f);
        A2[s] = v ? A * kLog2e : 0.0f;
        An[s] = A;
        Ainv[s] = 1.0f / A;
        if constexpr (DISC == DISC_CONST) am1[s] = expm1f(A);   // a - 1
    }
#pragma unroll
    for (int s = 0; s < SPL; ++s) asm volatile("" : "+v"(h[s]) : "v"(A2[s]));

    const float dtb = (DISC != DISC_CONST && p.dt_bias) ? p.dt_bias[tdc] : 0.0f;
    const float Dd = p.Dskip ? p.Dskip[tdc] : 0.0f;
    float wk[8], cb = 0.0f;
    const int W = p.W;
    if constexpr (CONV) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kk = i - (8 - W);
            wk[i] = (kk >= 0) ? p.conv_w[tdc * W + kk] : 0.0f;
        }
        cb = p.conv_b ? p.conv_b[tdc] : 0.0f;
    }
    // conv input before the chunk: x for t >= 0, else the carried history
    auto x_before = [&](int64_t tt) -> float {
        if (tt >= 0) return to_f32(X[(b * L + tt) * D + tdc]);
        if (p.conv_hist != nullptr && tt >= -(int64_t)(W - 1))
            return p.conv_hist[(b * (W - 1) + (W - 1) + tt) * D + tdc];
        return 0.0f;
    };

    RawTile<IOT, NP> raw;
    FetchOff fo;
    {
        const uint32_t es = sizeof(IOT);
        fo.x0 = (uint32_t)((rp * kRows) * (int)D + (int)tdc) * es;
        fo.xrow = (uint32_t)D * es;
        fo.bc0 = (uint32_t)((tid / NP) * (int)N + tid % NP) * es;
        fo.bcstep = (uint32_t)((kThreads / NP) * (int)N) * es;
    }

    // Per-(token, channel) quantities, once per tile element.
    auto transform = [&](int nv) {
        float uu[kRows];
        if constexpr (CONV) {
            // taps right-aligned in 8 slots; with a known width only the
            // last CW are nonzero (the zero taps add exactly nothing)
            constexpr int K0 = CW > 0 ? 8 - CW : 0;
            float win[kRows + 7 - K0];
#pragma unroll
            for (int i = 0; i < kRows + 7 - K0; ++i) win[i] = s_x[(rp * kRows + 1 + K0 + i) * kXS + tc];
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                float acc = cb;
#pragma unroll
                for (int kk = K0; kk < 8; ++kk) acc = fmaf(wk[kk], win[i + kk - K0], acc);
                uu[i] = silu_f(acc);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kRows; ++i) uu[i] = raw.f(raw.x[i]);
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int row = rp * kRows + i;
            const float dl = (DISC == DISC_CONST) ? 1.0f : softplus_f(raw.f(raw.dt[i]) + dtb);
            s_dl[tc][row] = make_float2(dl, (DISC == DISC_DB) ? dl * uu[i] : uu[i]);
            if constexpr (FINAL)
                s_gd[tc][row] = make_float2((Z != nullptr) ? silu_f(raw.f(raw.z[i])) : 1.0f, Dd * uu[i]);
        }
        (void)nv;
    };

    auto stage_x = [&]() {
        if constexpr (CONV) {
#pragma unroll
            for (int i = 0; i < kRows; ++i) s_x[(8 + rp * kRows + i) * kXS + tc] = raw.f(raw.x[i]);
        }
    };
    auto stage = [&](int it) {
        const int64_t ts = t0 + (int64_t)it * T;
        const int nv = (int)min((int64_t)T, t1 - ts);
        store_bc<IOT, NP, FINAL>(raw, s_B, s_C, tid, N);
        transform(nv);
        __syncthreads();
    };

    auto fetch = [&](int it) {
        const int64_t ts = t0 + (int64_t)it * T;
        load_raw<IOT, NP, FINAL, DISC != DISC_CONST>(raw, fo, X, DT, Z, Bp, Cp, b, L, D, N, ts);
    };

    float ssum = 0.0f;
    // one token (tail of the last tile)
    auto scan_step = [&](int t) {
        const float2 pk = s_dl[ch][t];
        const float dl = pk.x;
        float part = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < SPL; ++s2) {
            const float bq = s_B[(n0 + s2) * kTS + t];
            if constexpr (DISC == DISC_CONST) {
                h[s2] += fmaf(am1[s2], h[s2], pk.y * bq);
            } else {
                const float a = hw_exp2(dl * A2[s2]);
                float w;
                if constexpr (DISC == DISC_DB)
                    w = pk.y * bq;
                else
                    w = expm1f(dl * An[s2]) * Ainv[s2] * bq * pk.y;
                h[s2] = fmaf(a, h[s2], w);
            }
            if constexpr (FINAL) part = fmaf(s_C[(n0 + s2) * kTS + t], h[s2], part);
        }
        if constexpr (FINAL) {
            // every lane of the channel writes it
            s_yp[wv][ch][t] = kBanks ? banks_sum(part) : (kRowsOfStates ? rows_sum(part) : group_sum<4>(part));
        } else {
            ssum += dl;
        }
    };
    // Sixteen tokens t0 .. t0+15.  B and C of a token are the same for every
    // lane that holds the same state: a 16-lane row in the row layout, a
    // 4-lane bank in the bank layout.  In the row layout lane k of a row
    // reads its state's B and C of token t0 + k once and token t0 + k takes
    // them from lane k with a row broadcast (DPP row_newbcast); in the bank
    // layout lane q of a bank reads tokens t0 + 4q .. 4q+3 and token
    // t0 + 4g + i takes element i of lane g with a bank broadcast (DPP
    // quad_perm).  The compiler folds either broadcast into the multiply that
    // consumes it.  Only (dt, dt*u), which differ per channel, are read from
    // LDS per token.  The bank layout reduces two groups of four tokens at a
    // time, interleaved, so its DPP reads need no wait states of their own.
    auto scan_block16 = [&](int t0) {
        constexpr int NV = kBanks ? 4 : SPL;
        float bv[NV], cv[NV];
        if constexpr (kBanks) {
            lds_read_k<4>(&s_B[n0 * kTS + t0 + 4 * q4], bv);
            lds_read_k<4>(&s_C[n0 * kTS + t0 + 4 * q4], cv);
        } else {
#pragma unroll
            for (int s2 = 0; s2 < SPL; ++s2) {
                bv[s2] = s_B[(n0 + s2) * kTS + t0 + ch];
                cv[s2] = s_C[(n0 + s2) * kTS + t0 + ch];
            }
        }
        auto bcast = [&](auto gi, const float(&v)[NV], int s2) -> float {
            constexpr int k = decltype(gi)::value;   // token t0 + k
            if constexpr (kBanks)
                return bank_bcast<k / 4>(v[k % 4]);
            else
                return row_bcast<k>(v[s2]);
        };
        float parts[4][4];
        static_for<4>([&](auto gI) {
            constexpr int g = decltype(gI)::value;
            const int t = t0 + 4 * g;
            float (&part)[4] = parts[g];
            const float4 d01 = *reinterpret_cast<const float4 *>(&s_dl[ch][t]);
            const float4 d23 = *reinterpret_cast<const float4 *>(&s_dl[ch][t + 2]);
            const float dl[4] = {d01.x, d01.z, d23.x, d23.z};
            const float dy[4] = {d01.y, d01.w, d23.y, d23.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) part[i] = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < SPL; ++s2) {
                static_for<4>([&](auto iI) {
                    constexpr int i = decltype(iI)::value;
                    const float bq = bcast(std::integral_constant<int, 4 * g + i>(), bv, s2);
                    const float a = hw_exp2(dl[i] * A2[s2]);
                    float w;
                    if constexpr (DISC == DISC_DB)
                        w = dy[i] * bq;
                    else
                        w = expm1f(dl[i] * An[s2]) * Ainv[s2] * bq * dy[i];
                    h[s2] = fmaf(a, h[s2], w);
                    // the first state's term is a product (a multiply takes the
                    // broadcast operand directly; fmaf(c, h, 0) does not)
                    const float cq = bcast(std::integral_constant<int, 4 * g + i>(), cv, s2);
                    part[i] = (s2 == 0) ? cq * h[s2] : fmaf(cq, h[s2], part[i]);
                });
            }
            if constexpr (!kBanks) {
                s_yp[wv][ch][t + j] = rows_transpose_sum(part);
            } else if constexpr (g % 2 == 1) {
                float ya, yb;
                banks_transpose_sum2(parts[g - 1], part, ya, yb);
                s_yp[wv][ch][t - 4 + j] = ya;
                s_yp[wv][ch][t + j] = yb;
            }
        });
    };
    // four tokens t .. t+3: 16-byte LDS reads, one transposed quad reduction
    auto scan_group = [&](int t) {
        const float4 d01 = *reinterpret_cast<const float4 *>(&s_dl[ch][t]);
        const float4 d23 = *reinterpret_cast<const float4 *>(&s_dl[ch][t + 2]);
        const float dl[4] = {d01.x, d01.z, d23.x, d23.z};
        const float dy[4] = {d01.y, d01.w, d23.y, d23.w};
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s2 = 0; s2 < SPL; ++s2) {
            const float4 b4 = *reinterpret_cast<const float4 *>(&s_B[(n0 + s2) * kTS + t]);
            const float bq[4] = {b4.x, b4.y, b4.z, b4.w};
            float cq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (FINAL) {
                const float4 c4 = *reinterpret_cast<const float4 *>(&s_C[(n0 + s2) * kTS + t]);
                cq[0] = c4.x; cq[1] = c4.y; cq[2] = c4.z; cq[3] = c4.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (DISC == DISC_CONST) {
                    h[s2] += fmaf(am1[s2], h[s2], dy[i] * bq[i]);
                } else {
                    const float a = hw_exp2(dl[i] * A2[s2]);
                    float w;
                    if constexpr (DISC == DISC_DB)
                        w = dy[i] * bq[i];
                    else
                        w = expm1f(dl[i] * An[s2]) * Ainv[s2] * bq[i] * dy[i];
                    h[s2] = fmaf(a, h[s2], w);
                }
                if constexpr (FINAL) part[i] = fmaf(cq[i], h[s2], part[i]);
            }
        }
        if constexpr (FINAL) {
            s_yp[wv][ch][t + j] = kBanks ? banks_transpose_sum(part)
                                         : (kRowsOfStates ? rows_transpose_sum(part) : quad_transpose_sum(part, j));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ssum += dl[i];
        }
    };

    constexpr int kHaloRp = (T - 8) / kRows;   // first thread row-group holding the last 8 rows
    if (ntiles > 0) {
        fetch(0);
        if constexpr (CONV) {
            if (rp == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) s_x[i * kXS + tc] = x_before(t0 - 8 + i);
            }
        }
        stage_x();
        __syncthreads();
        stage(0);
        if (ntiles > 1) fetch(1);
    }
    // Two barriers per tile.  The first ends the scan of tile it (its readout
    // partials are complete) and publishes the next tile's raw conv rows,
    // written after the scan; the second publishes the next tile's B, C and
    // transformed rows, written after the readout.
    for (int it = 0; it < ntiles; ++it) {
        const int64_t ts = t0 + (int64_t)it * T;
        const int nv = (int)min((int64_t)T, t1 - ts);
        if (nv == T) {
            if constexpr (FINAL && kRowsOfStates) {
#pragma unroll
                for (int t = 0; t < T; t += 16) scan_block16(t);
            } else {
#pragma unroll
                for (int t = 0; t < T; t += 4) scan_group(t);
            }
        } else {
            int t = 0;
            for (; t + 4 <= nv; t += 4) scan_group(t);
            for (; t < nv; ++t) scan_step(t);
        }
        if (it + 1 < ntiles) {
            if constexpr (CONV) {
                // the last 8 rows become the next tile's history rows; each
                // thread moves the rows it staged itself (no other thread
                // touches them before the next barrier)
                if (rp >= kHaloRp) {
#pragma unroll
                    for (int i = 0; i < kRows; ++i)
                        s_x[(rp * kRows + i - (T - 8)) * kXS + tc] = s_x[(8 + rp * kRows + i) * kXS + tc];
                }
            }
            stage_x();
        }
        __syncthreads();
        // readout: ((w0 + w1) + (w2 + w3)) + Dskip*u, then the gate
        float yo[kRows];
        if constexpr (FINAL) {
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                const int row = rp * kRows + i;
                const float2 gd = s_gd[tc][row];
                const float ys = (s_yp[0][tc][row] + s_yp[1][tc][row]) + (s_yp[2][tc][row] + s_yp[3][tc][row]);
                yo[i] = (ys + gd.y) * gd.x;
            }
        }
        // A wait for loaded data also waits for every store in flight, so y
        // is stored after the next tile is staged and the one after it is
        // requested (whose waits would otherwise hold for these stores), and
        // has a whole tile of scanning to drain.
        // (the descriptor's range ends at the tile's last valid row, so rows
        // past it are dropped by the hardware)
        auto store_y = [&]() {
            if constexpr (FINAL) {
                const buf_t rY = make_buf(Y + (b * L + ts) * D, (uint64_t)nv * D * sizeof(IOT));
                if (tvalid) {
#pragma unroll
                    for (int i = 0; i < kRows; ++i) buf_st(rY, fo.x0 + (uint32_t)i * fo.xrow, Y, yo[i]);
                }
            }
        };
        if (it + 1 < ntiles) {
            stage(it + 1);
            if (it + 2 < ntiles) fetch(it + 2);
            store_y();
        } else {
            store_y();
        }
    }

    if constexpr (FINAL) {
        if (k == p.K - 1) {
            if (dvalid && p.hT != nullptr && nvalid > 0)
                store_k<SPL>(p.hT + (b * D + d) * N + n0, h, nvalid, vecN && (SPL % 4 == 0));
            if constexpr (CONV) {
                if (p.conv_state_out != nullptr && rp == 0 && tvalid) {
                    // the last W-1 conv inputs: staged rows of the last tile, or
                    // the carried history when the sequence is empty
                    const int64_t tl = t0 + (int64_t)max(ntiles - 1, 0) * T;
                    for (int jj = 0; jj < W - 1; ++jj) {
                        const int64_t tt = L - (W - 1) + jj;
                        const float v = (ntiles > 0) ? s_x[(int)(tt - (tl - 8)) * kXS + tc] : x_before(tt);
                        p.conv_state_out[(b * (W - 1) + jj) * D + td] = v;
                    }
                }
            }
        }
    } else {
        if (dvalid) {
            const int64_t o = (b * p.K + k) * D + d;
            if (nvalid > 0) store_k<SPL>(p.agg_h + o * N + n0, h, nvalid, vecN && (SPL % 4 == 0));
            if (wv == 0 && j == 0) p.agg_s[o] = ssum;
        }
    }
}

// Walks the chunks of every (b, d, n) in time order, replacing each chunk's
// local end state by the exact state at the chunk's start.  The chunk's
// decay e^(A S_k) enters in complement form, H + (expm1(A S_k) H + W_k), which
// keeps short chunks of slow decays accurate.  Also copies the
// incoming conv history so that MODE_FINAL never reads a buffer the same
// launch writes.
__global__ __launch_bounds__(256) void carry_kernel(const float *A_log, const float *h0, float *agg_h,
                                                    const float *agg_s, int64_t B, int64_t D,
                                                    int64_t N, int K, const float *conv_in,
                                                    float *conv_copy, int64_t conv_count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = B * D * N;
    if (i < total) {
        const int64_t n = i % N, d = (i / N) % D, b = i / (N * D);
        const float A = neg_exp_f(A_log[d * N + n]);
        float H = h0 ? h0[i] : 0.0f;
        // Eight chunks' summaries are loaded before their links of the chain
        // are taken: loaded one at a time, each load would wait for the store
        // before it (the compiler cannot tell them apart).
        for (int k0 = 0; k0 < K; k0 += 8) {
            float Wv[8], Sv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = k0 + j;
                Wv[j] = k < K ? agg_h[((b * K + k) * D + d) * N + n] : 0.0f;
                Sv[j] = k + 1 < K ? agg_s[(b * K + k) * D + d] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = k0 + j;
                if (k < K) {
                    agg_h[((b * K + k) * D + d) * N + n] = H;
                    if (k + 1 < K) H += fmaf(expm1f(A * Sv[j]), H, Wv[j]);
                }
            }
        }
    }
    if (conv_in != nullptr)
        for (int64_t j = i; j < conv_count; j += (int64_t)gridDim.x * blockDim.x) conv_copy[j] = conv_in[j];
}

// ------------------------------------------------ one-wavefront chunk scan
// A split in time (above) supplies the parallelism of long sequences, so
// their chunks run in single-wavefront workgroups with four states per lane
// and no workgroup barrier.  Used for N = 16, no fused conv, the dt*B and ZOH
// forms, and D a multiple of 16.  The wavefront owns 16 channels of one
// batch row and one chunk:
//  - scan role: lane (ch, r) = (lane & 15, lane >> 4) keeps states
//    4r .. 4r+3 of channel ch.  A 16-lane row shares its states over sixteen
//    channels, so the B and C of token t0 + kk reach the row from lane kk by
//    DPP row broadcast; lane (kk, r) loads B[t0 + kk][4r .. 4r+3] (and C)
//    straight from memory, 16 tokens x 16 states contiguous per wavefront;
//  - io role: lane (cp, rq) = (lane & 7, lane >> 3) loads, transforms and
//    stores channels 2cp and 2cp+1 of tokens rq + 8i, two channels per access;
//  - the per-token transform (softplus, dt*u, the gate, D*u) goes from the io
//    role to the scan role through LDS, [channel][token];
//  - the readout adds a lane's four states in registers and the four rows
//    with the row swaps, leaving token t + r of channel ch in lane (ch, r),
//    which finishes y; y goes back to the io role through LDS for the store.
// Tiles are 32 tokens; the next tile's loads are issued before the current
// tile's scan, and the current tile's stores after them.  Tokens past the
// chunk get dt = dt*u = 0, which leaves the state unchanged, and are not
// stored.
constexpr int kLT = 32;            // tokens per tile
constexpr int kLDP = kLT + 2;      // padded [channel][token] row of float2
constexpr int kLYS = 18;           // [token][channel] row of the y tile

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Two adjacent channels of one token (io role) and four adjacent states of one
// token (B, C), as raw io bits, with their conversions.
template <typename IOT> struct LongIO;
template <> struct LongIO<float> {
    typedef u32x2 pair_t;
    typedef u32x4 quad_t;
    __device__ __forceinline__ static pair_t ld2(buf_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0); }
    __device__ __forceinline__ static quad_t ld4(buf_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0); }
    __device__ __forceinline__ static float e2(pair_t v, int c) { return __uint_as_float(c ? v.y : v.x); }
    __device__ __forceinline__ static float e4(quad_t v, int s) {
        return __uint_as_float(s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w);
    }
    __device__ __forceinline__ static void st2(buf_t r, uint32_t o, float a, float b) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(a), __float_as_uint(b)}, r, o, 0, 0);
    }
};
template <> struct LongIO<bf16_t> {
    typedef uint32_t pair_t;
    typedef u32x2 quad_t;
    __device__ __forceinline__ static pair_t ld2(buf_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0); }
    __device__ __forceinline__ static quad_t ld4(buf_t r, uint32_t o) { return __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0); }
    __device__ __forceinline__ static float e2(pair_t v, int c) { return __uint_as_float(c ? (v & 0xffff0000u) : (v << 16)); }
    __device__ __forceinline__ static float e4(quad_t v, int s) {
        const uint32_t w = s < 2 ? v.x : v.y;
        return __uint_as_float((s & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ __forceinline__ static void st2(buf_t r, uint32_t o, float a, float b) {
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)bf16_rne(a) | ((uint32_t)bf16_rne(b) << 16), r, o, 0, 0);
    }
};


template <typename IOT, int DISC, int MODE>
__global__ __launch_bounds__(64) void scan_long_kernel(FwdParams p) {
    constexpr int T = kLT;
    constexpr bool FINAL = MODE == MODE_FINAL;
    typedef LongIO<IOT> IO;
    __shared__ __align__(16) float2 s_dl[16][kLDP];                  // {dt, dt*u} (ZOH: {dt, u})
    __shared__ __align__(16) float2 s_gd[FINAL ? 16 : 1][kLDP];      // {gate, Dskip*u}
    __shared__ __align__(16) float s_y[FINAL ? T : 1][kLYS];

    const IOT *X = static_cast<const IOT *>(p.x);
    const IOT *DT = static_cast<const IOT *>(p.dt);
    const IOT *Bp = static_cast<const IOT *>(p.Bm);
    const IOT *Cp = static_cast<const IOT *>(p.Cm);
    const IOT *Z = FINAL ? static_cast<const IOT *>(p.z) : nullptr;
    IOT *Y = static_cast<IOT *>(p.y);

    const int lane = threadIdx.x;
    const int64_t bid = xcd_remap((int64_t)blockIdx.x, (int64_t)gridDim.x, kNumXcd);
    const int64_t g = bid % p.groups;
    const int64_t rest = bid / p.groups;
    const int k = (int)(rest % p.Kgrid);
    const int64_t b = rest / p.Kgrid;
    const int64_t D = p.D, L = p.L;
    const int64_t d0 = g * 16;
    const int64_t t0 = (int64_t)k * p.chunk;
    const int64_t t1 = min(L, t0 + p.chunk);
    const int ntiles = (int)((t1 - t0 + T - 1) / T);

    const int ch = lane & 15, r = lane >> 4;     // scan role
    const int cp = lane & 7, rq = lane >> 3;     // io role
    const int64_t d = d0 + ch;
    const uint32_t es = sizeof(IOT);

    float h[4] = {0.0f, 0.0f, 0.0f, 0.0f}, A2[4], An[4], Ainv[4];
    if (p.init != nullptr) {
        const float4 v = *reinterpret_cast<const float4 *>(p.init + b * p.init_bstride + (int64_t)k * p.init_kstride +
                                                           d * 16 + 4 * r);
        h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
    }
    {
        const float4 al = *reinterpret_cast<const float4 *>(p.A_log + d * 16 + 4 * r);
        const float alv[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const float A = neg_exp_f(alv[s2]);
            A2[s2] = A * kLog2e;
            An[s2] = A;
            Ainv[s2] = 1.0f / A;
        }
    }
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) asm volatile("" : "+v"(h[s2]) : "v"(A2[s2]));
    float dtb[2], Dd[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        dtb[c] = p.dt_bias ? p.dt_bias[d0 + 2 * cp + c] : 0.0f;
        Dd[c] = (FINAL && p.Dskip) ? p.Dskip[d0 + 2 * cp + c] : 0.0f;
    }

    // one tile's raw loads (io role: x, dt, z; scan role: B, C of two 16-token blocks)
    typename IO::pair_t rx[4], rdt[4], rz[4];
    typename IO::quad_t rB[2], rC[2];
    const uint32_t xo = (uint32_t)((int64_t)rq * D + 2 * cp) * es;    // + i * 8 rows
    const uint32_t xs = (uint32_t)(8 * D) * es;
    const uint32_t bo = (uint32_t)(ch * 16 + 4 * r) * es;              // + j * 16 tokens
    const uint32_t bs = (uint32_t)(16 * 16) * es;
    auto fetch = [&](int it) {
        const int64_t ts = t0 + (int64_t)it * T;
        const int64_t left = t1 - ts;
        const uint64_t xr = (uint64_t)(left * D - d0) * es;
        const buf_t bX = make_buf(X + (b * L + ts) * D + d0, xr);
        const buf_t bD = make_buf(DT + (b * L + ts) * D + d0, xr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rx[i] = IO::ld2(bX, xo + i * xs);
            rdt[i] = IO::ld2(bD, xo + i * xs);
        }
        if (Z != nullptr) {
            const buf_t bZ = make_buf(Z + (b * L + ts) * D + d0, xr);
#pragma unroll
            for (int i = 0; i < 4; ++i) rz[i] = IO::ld2(bZ, xo + i * xs);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) rz[i] = typename IO::pair_t{};
        }
        const uint64_t br = (uint64_t)(left * 16) * es;
        const buf_t bB = make_buf(Bp + (b * L + ts) * 16, br);
#pragma unroll
        for (int j = 0; j < 2; ++j) rB[j] = IO::ld4(bB, bo + j * bs);
        if constexpr (FINAL) {
            const buf_t bC = make_buf(Cp + (b * L + ts) * 16, br);
#pragma unroll
            for (int j = 0; j < 2; ++j) rC[j] = IO::ld4(bC, bo + j * bs);
        }
    };

    float ssum = 0.0f;
    float bv[2][4], cv[2][4];
    if (ntiles > 0) fetch(0);
    for (int it = 0; it < ntiles; ++it) {
        const int64_t ts = t0 + (int64_t)it * T;
        const int nv = (int)min((int64_t)T, t1 - ts);
        // transform (io role) into LDS; B, C out of the raw registers
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = rq + 8 * i;
            const bool v = tt < nv;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float u = IO::e2(rx[i], c);
                const float dl = v ? softplus_f(IO::e2(rdt[i], c) + dtb[c]) : 0.0f;
                const float dy = (DISC == DISC_DB) ? dl * u : (v ? u : 0.0f);
                s_dl[2 * cp + c][tt] = make_float2(dl, dy);
                if constexpr (FINAL)
                    s_gd[2 * cp + c][tt] = make_float2((Z != nullptr) ? silu_f(IO::e2(rz[i], c)) : 1.0f, Dd[c] * u);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                bv[j][s2] = IO::e4(rB[j], s2);
                cv[j][s2] = FINAL ? IO::e4(rC[j], s2) : 0.0f;
            }
        if (it + 1 < ntiles) fetch(it + 1);
        __syncthreads();
        // scan role: two blocks of 16 tokens
        static_for<2>([&](auto jI) {
            constexpr int j = decltype(jI)::value;
            static_for<4>([&](auto gI) {
                constexpr int g4 = decltype(gI)::value;
                const int t = 16 * j + 4 * g4;
                const float4 d01 = *reinterpret_cast<const float4 *>(&s_dl[ch][t]);
                const float4 d23 = *reinterpret_cast<const float4 *>(&s_dl[ch][t + 2]);
                const float dl[4] = {d01.x, d01.z, d23.x, d23.z};
                const float dy[4] = {d01.y, d01.w, d23.y, d23.w};
                float part[4];
                static_for<4>([&](auto iI) {
                    constexpr int i = decltype(iI)::value;
                    constexpr int kk = 4 * g4 + i;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        const float bq = row_bcast<kk>(bv[j][s2]);
                        const float a = hw_exp2(dl[i] * A2[s2]);
                        float w;
                        if constexpr (DISC == DISC_DB)
                            w = dy[i] * bq;
                        else
                            w = expm1f(dl[i] * An[s2]) * Ainv[s2] * bq * dy[i];
                        h[s2] = fmaf(a, h[s2], w);
                        if constexpr (FINAL)
                            part[i] = (s2 == 0) ? row_bcast<kk>(cv[j][s2]) * h[s2]
                                                : fmac_row_bcast<kk>(part[i], cv[j][s2], h[s2]);
                    }
                });
                if constexpr (FINAL) {
                    // token t + r of channel ch, over all sixteen states
                    const float ys = rows_transpose_sum(part);
                    const float2 gd = s_gd[ch][t + r];
                    s_y[t + r][ch] = (ys + gd.y) * gd.x;
                } else {
                    ssum += (dl[0] + dl[1]) + (dl[2] + dl[3]);
                }
            });
        });
        if constexpr (FINAL) {
            __syncthreads();
            const buf_t bY = make_buf(Y + (b * L + ts) * D + d0, (uint64_t)((int64_t)nv * D - d0) * es);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = rq + 8 * i;
                IO::st2(bY, xo + i * xs, s_y[tt][2 * cp], s_y[tt][2 * cp + 1]);
            }
        }
    }

    if constexpr (FINAL) {
        if (k == p.K - 1 && p.hT != nullptr)
            *reinterpret_cast<float4 *>(p.hT + (b * D + d) * 16 + 4 * r) = make_float4(h[0], h[1], h[2], h[3]);
    } else {
        const int64_t o = (b * p.K + k) * D + d;
        *reinterpret_cast<float4 *>(p.agg_h + o * 16 + 4 * r) = make_float4(h[0], h[1], h[2], h[3]);
        if (r == 0) p.agg_s[o] = ssum;
    }
}

template <typename IOT, int SPL, int DISC, bool CONV, int MODE>
hipError_t launch_one(const FwdParams &p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.groups * p.Kgrid * p.B;
    if (blocks <= 0) return hipSuccess;
    // the 4-tap conv of the Mamba blocks gets its own instance
    if (CONV && p.W == 4)
        hipLaunchKernelGGL((scan_fwd_kernel<IOT, SPL, DISC, CONV, MODE, 4>),
                           dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((scan_fwd_kernel<IOT, SPL, DISC, CONV, MODE>),
                           dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename IOT, int SPL>
hipError_t dispatch_mode(const FwdParams &p, int disc, bool conv, int mode, hipStream_t s) {
#define SSM_FWD_CASE(DI, CV, MO)                                                   \
    if (disc == DI && conv == CV && mode == MO) return launch_one<IOT, SPL, DI, CV, MO>(p, s);
    SSM_FWD_CASE(DISC_DB, false, MODE_FINAL)
    SSM_FWD_CASE(DISC_DB, true, MODE_FINAL)
    SSM_FWD_CASE(DISC_DB, false, MODE_LOCAL)
    SSM_FWD_CASE(DISC_DB, true, MODE_LOCAL)
    SSM_FWD_CASE(DISC_ZOH, false, MODE_FINAL)
    SSM_FWD_CASE(DISC_ZOH, true, MODE_FINAL)
    SSM_FWD_CASE(DISC_ZOH, false, MODE_LOCAL)
    SSM_FWD_CASE(DISC_ZOH, true, MODE_LOCAL)
    SSM_FWD_CASE(DISC_CONST, false, MODE_FINAL)
    SSM_FWD_CASE(DISC_CONST, true, MODE_FINAL)
    SSM_FWD_CASE(DISC_CONST, false, MODE_LOCAL)
    SSM_FWD_CASE(DISC_CONST, true, MODE_LOCAL)
#undef SSM_FWD_CASE
    return hipErrorInvalidValue;
}

template <typename IOT>
hipError_t dispatch_spl(const FwdParams &p, int disc, bool conv, int mode, hipStream_t s) {
    if (p.N <= 16) return dispatch_mode<IOT, 1>(p, disc, conv, mode, s);
    if (p.N <= 32) return dispatch_mode<IOT, 2>(p, disc, conv, mode, s);
    return dispatch_mode<IOT, 4>(p, disc, conv, mode, s);
}

hipError_t dispatch(const FwdParams &p, int bf16, int disc, bool conv, int mode, hipStream_t s) {
    if (bf16) return dispatch_spl<bf16_t>(p, disc, conv, mode, s);
    return dispatch_spl<float>(p, disc, conv, mode, s);
}

// The one-wavefront chunk scan covers N = 16, no fused conv, the input-driven
// decay, and whole 16-channel groups.
bool long_ok(int64_t D, int64_t N, int W, int disc) {
    return N == 16 && W == 0 && (disc == DISC_DB || disc == DISC_ZOH) && D % 16 == 0;
}

template <typename IOT, int DISC>
hipError_t launch_long_t(const FwdParams &p, int mode, hipStream_t s) {
    const int64_t blocks = (int64_t)p.groups * p.Kgrid * p.B;
    if (blocks <= 0) return hipSuccess;
    if (mode == MODE_FINAL)
        hipLaunchKernelGGL((scan_long_kernel<IOT, DISC, MODE_FINAL>), dim3((unsigned)blocks), dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL((scan_long_kernel<IOT, DISC, MODE_LOCAL>), dim3((unsigned)blocks), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t dispatch_long(const FwdParams &p, int bf16, int disc, int mode, hipStream_t s) {
    if (bf16) return disc == DISC_DB ? launch_long_t<bf16_t, DISC_DB>(p, mode, s)
                                     : launch_long_t<bf16_t, DISC_ZOH>(p, mode, s);
    return disc == DISC_DB ? launch_long_t<float, DISC_DB>(p, mode, s) : launch_long_t<float, DISC_ZOH>(p, mode, s);
}

struct FwdWs {
    float *agg_h, *agg_s, *conv_copy;
};

FwdWs carve(void *ws, int64_t B, int64_t D, int64_t N, int W, int K) {
    char *base = static_cast<char *>(ws);
    FwdWs r;
    r.agg_h = reinterpret_cast<float *>(base);
    base += ws_align(sizeof(float) * (size_t)(B * K * D * N));
    r.agg_s = reinterpret_cast<float *>(base);
    base += ws_align(sizeof(float) * (size_t)(B * K * D));
    r.conv_copy = reinterpret_cast<float *>(base);
    (void)W;
    return r;
}

int64_t num_chunks(int64_t L, int64_t chunk) {
    if (L <= 0 || chunk >= L) return 1;
    return (L + chunk - 1) / chunk;
}

}  // namespace

int64_t scan_fwd_auto_chunk(int64_t B, int64_t L, int64_t D, int64_t N, int W, int disc) {
    const int64_t blocks = B * ((D + kCPW - 1) / kCPW);
    if (long_ok(D, N, W, disc) && blocks <= 256 && L >= 512) {
        // one-wavefront chunks: at most three wavefronts per SIMD (1024 SIMDs;
        // a grid past a whole number of wavefronts per SIMD leaves some SIMDs
        // a round behind, so the count rounds down), chunks of at least 256
        // tokens, a multiple of 64
        int64_t K = 3072 / blocks;
        K = std::min<int64_t>(K, L / 256);
        if (K > 1) {
            int64_t chunk = (L + K - 1) / K;
            chunk = (chunk + 63) / 64 * 64;
            if (chunk < L) return chunk;
        }
    }
    // aim for three four-wavefront blocks per CU (256 CUs)
    if (blocks >= 512 || L <= 2 * kTile) return L > 0 ? L : 1;
    int64_t K = (768 + blocks - 1) / blocks;
    K = std::min<int64_t>(K, (L + 4 * kTile - 1) / (4 * kTile));
    if (K <= 1) return L;
    int64_t chunk = (L + K - 1) / K;
    chunk = (chunk + kTile - 1) / kTile * kTile;
    return chunk;
}

size_t scan_fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int W, int64_t chunk_len) {
    const int64_t K = num_chunks(L, chunk_len);
    if (K <= 1) return 0;
    return ws_align(sizeof(float) * (size_t)(B * K * D * N)) + ws_align(sizeof(float) * (size_t)(B * K * D)) +
           ws_align(sizeof(float) * (size_t)(B * (W > 1 ? W - 1 : 0) * D));
}

hipError_t launch_scan_chunk_starts(const ScanFwdArgs &a, int64_t chunk, float *agg_h, float *agg_s,
                                   hipStream_t s) {
    FwdParams p{};
    p.x = a.x; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log;
    p.Bm = a.Bm; p.Cm = a.Cm; p.Dskip = nullptr; p.z = nullptr;
    p.conv_w = a.conv_w; p.conv_b = a.conv_b;
    p.B = a.B; p.L = a.L; p.D = a.D; p.N = a.N; p.W = a.W;
    p.groups = (int)((a.D + kCPW - 1) / kCPW);
    const int64_t K = num_chunks(a.L, chunk);
    if (K <= 1) return hipErrorInvalidValue;
    p.chunk = chunk;
    p.K = (int)K;
    p.agg_h = agg_h; p.agg_s = agg_s;
    p.Kgrid = (int)K - 1;
    p.conv_hist = a.conv_state_in;
    hipError_t e = long_ok(a.D, a.N, a.W, a.disc) ? dispatch_long(p, a.bf16, a.disc, MODE_LOCAL, s)
                                                  : dispatch(p, a.bf16, a.disc, a.W > 0, MODE_LOCAL, s);
    if (e != hipSuccess) return e;
    const int64_t total = a.B * a.D * a.N;
    hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a.A_log, a.h0,
                       agg_h, agg_s, a.B, a.D, a.N, (int)K, nullptr, nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_scan_fwd(const ScanFwdArgs &a, hipStream_t s) {
    FwdParams p{};
    p.x = a.x; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log;
    p.Bm = a.Bm; p.Cm = a.Cm; p.Dskip = a.Dskip; p.z = a.z;
    p.conv_w = a.conv_w; p.conv_b = a.conv_b;
    p.conv_state_out = a.conv_state_out;
    p.hT = a.hT; p.y = a.y;
    p.B = a.B; p.L = a.L; p.D = a.D; p.N = a.N; p.W = a.W;
    p.groups = (int)((a.D + kCPW - 1) / kCPW);
    const bool conv = a.W > 0;
    const int64_t K = num_chunks(a.L, a.chunk_len);
    if (K <= 1) {
        p.chunk = a.L > 0 ? a.L : 1;
        p.K = 1; p.Kgrid = 1;
        p.init = a.h0; p.init_bstride = a.D * a.N; p.init_kstride = 0;
        p.conv_hist = a.conv_state_in;
        return dispatch(p, a.bf16, a.disc, conv, MODE_FINAL, s);
    }
    FwdWs w = carve(a.ws, a.B, a.D, a.N, a.W, (int)K);
    p.chunk = a.chunk_len;
    p.K = (int)K;
    p.agg_h = w.agg_h; p.agg_s = w.agg_s;
    // level 1: local scans of chunks 0 .. K-2 (the last chunk's summary is unused)
    p.Kgrid = (int)K - 1;
    p.init = nullptr; p.init_bstride = 0; p.init_kstride = 0;
    p.conv_hist = a.conv_state_in;
    const bool lng = long_ok(a.D, a.N, a.W, a.disc);
    hipError_t e = lng ? dispatch_long(p, a.bf16, a.disc, MODE_LOCAL, s)
                       : dispatch(p, a.bf16, a.disc, conv, MODE_LOCAL, s);
    if (e != hipSuccess) return e;
    // level 2: carries across chunks
    const int64_t total = a.B * a.D * a.N;
    const int64_t conv_count = (conv && a.conv_state_in && a.W > 1) ? a.B * (a.W - 1) * a.D : 0;
    const int64_t threads = std::max(total, conv_count);
    hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a.A_log,
                       a.h0, w.agg_h, w.agg_s, a.B, a.D, a.N, (int)K,
                       conv_count ? a.conv_state_in : nullptr, w.conv_copy, conv_count);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // fix-up: every chunk re-scanned from its exact starting state
    p.Kgrid = (int)K;
    p.init = w.agg_h; p.init_bstride = K * a.D * a.N; p.init_kstride = a.D * a.N;
    p.conv_hist = conv_count ? w.conv_copy : nullptr;
    return lng ? dispatch_long(p, a.bf16, a.disc, MODE_FINAL, s) : dispatch(p, a.bf16, a.disc, conv, MODE_FINAL, s);
}

}  // namespace ssm
