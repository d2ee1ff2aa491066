// abi.cpp -- the library's C ABI (include/ssm.h): argument validation on the
// host, before any HIP call, then dispatch to the kernel launchers.
#include "ssm.h"

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "launch.hpp"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // per tensor

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t io_size(int32_t io) { return io == SSM_BF16 ? 2 : 4; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > kMaxElems / a) return false;
    *out = a * b;
    return true;
}

bool elems(std::initializer_list<int64_t> dims, int64_t *out) {
    int64_t n = 1;
    for (int64_t d : dims)
        if (!mul_ok(n, d, &n)) return false;
    *out = n;
    return true;
}

// The largest launch grid (in workgroups, or 256-thread groups) any kernel of
// the library takes; shapes that would need more are rejected with
// SSM_ERR_BAD_SHAPE before any HIP call (kernels index rows and workgroups in
// 32 bits).
constexpr int64_t kMaxGrid = 0x7fffffff;
bool grid_ok(std::initializer_list<int64_t> dims) {
    int64_t n;
    return elems(dims, &n) && n <= kMaxGrid;
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Range {
    const void *p;
    int64_t bytes;
};

bool overlap(const Range &a, const Range &b) {
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Every output must be disjoint from every input and every other output,
// except the listed exact in-place pairs (same pointer, same size).
struct AliasCheck {
    std::vector<Range> ins, outs;
    std::vector<std::pair<const void *, const void *>> allowed;
    bool ok() const {
        for (size_t i = 0; i < outs.size(); ++i) {
            for (const Range &r : ins) {
                if (!overlap(outs[i], r)) continue;
                bool exact = false;
                for (auto &pr : allowed)
                    if (pr.first == r.p && pr.second == outs[i].p && r.p == outs[i].p &&
                        r.bytes == outs[i].bytes)
                        exact = true;
                if (!exact) return false;
            }
            for (size_t j = i + 1; j < outs.size(); ++j)
                if (overlap(outs[i], outs[j])) return false;
        }
        return true;
    }
};

ssm_status hip_status(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

bool valid_io(int32_t io) { return io == SSM_F32 || io == SSM_BF16; }
bool valid_disc(int32_t d) { return d == SSM_DISC_DELTA_B || d == SSM_DISC_ZOH || d == SSM_DECAY_CONST; }
bool has_step_size(int32_t d) { return d != SSM_DECAY_CONST; }

ssm_status check_scan_desc(const ssm_scan_desc *d) {
    if (!d) return SSM_ERR_NULL_ARG;
    if (!valid_io(d->io_dtype) || !valid_disc(d->disc)) return SSM_ERR_UNSUPPORTED;
    if (d->batch < 1 || d->seqlen < 0 || d->dim < 1 || d->dim > SSM_MAX_SCAN_DIM || d->dstate < 1 ||
        d->dstate > SSM_MAX_DSTATE)
        return SSM_ERR_BAD_SHAPE;
    if (d->conv_width < 0 || d->conv_width > SSM_MAX_CONV_WIDTH) return SSM_ERR_BAD_SHAPE;
    if (d->chunk_len < -1) return SSM_ERR_BAD_SHAPE;
    int64_t n;
    if (!elems({d->batch, d->seqlen, d->dim}, &n) || !elems({d->batch, d->seqlen, d->dstate}, &n) ||
        !elems({d->batch, d->dim, d->dstate}, &n))
        return SSM_ERR_BAD_SHAPE;
    return SSM_OK;
}

int64_t resolve_chunk(const ssm_scan_desc *d) {
    const int64_t L = d->seqlen;
    if (d->chunk_len == -1 || L <= 1) return std::max<int64_t>(L, 1);
    if (d->chunk_len > 0) return std::min<int64_t>(d->chunk_len, L);
    return ssm::scan_fwd_auto_chunk(d->batch, L, d->dim, d->dstate, d->conv_width, d->disc);
}

}  // namespace

extern "C" {

int32_t ssm_version(void) { return SSM_ABI_VERSION * 100 + 1; }

const char *ssm_status_string(ssm_status s) {
    switch (s) {
        case SSM_OK: return "success";
        case SSM_ERR_NULL_ARG: return "a required pointer is NULL";
        case SSM_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
        case SSM_ERR_UNSUPPORTED: return "request not supported by this library";
        case SSM_ERR_WORKSPACE: return "workspace missing or smaller than the queried size";
        case SSM_ERR_ALIGNMENT: return "a tensor does not start on a 16-byte boundary";
        case SSM_ERR_ALIAS: return "buffers overlap in a way the call does not allow";
        case SSM_ERR_HIP: return "a HIP launch failed";
        case SSM_ERR_SCRATCH_LIMIT: return "the request needs more than the library's static scratch buffer holds";
        default: return "unknown status";
    }
}

ssm_status conv1d_causal(const ssm_conv_desc *desc, const void *x, const float *w, const float *b,
                         const float *state_in, float *state_out, void *y, void *stream) {
    if (!desc) return SSM_ERR_NULL_ARG;
    if (!valid_io(desc->io_dtype) || desc->reserved != 0 || (desc->fuse_silu != 0 && desc->fuse_silu != 1))
        return SSM_ERR_UNSUPPORTED;
    if (desc->batch < 1 || desc->seqlen < 0 || desc->dim < 1 || desc->width < 1 ||
        desc->width > SSM_MAX_CONV_WIDTH)
        return SSM_ERR_BAD_SHAPE;
    const int64_t B = desc->batch, L = desc->seqlen, D = desc->dim, W = desc->width;
    int64_t nx, nst;
    if (!elems({B, L, D}, &nx) || !elems({B, W - 1, D}, &nst)) return SSM_ERR_BAD_SHAPE;
    if (!grid_ok({B, std::max<int64_t>(L, 1), cdiv(D, 256)})) return SSM_ERR_BAD_SHAPE;
    if (!w || (L > 0 && (!x || !y))) return SSM_ERR_NULL_ARG;
    for (const void *p : {(const void *)x, (const void *)w, (const void *)b, (const void *)state_in,
                          (const void *)state_out, (const void *)y})
        if (!aligned16(p)) return SSM_ERR_ALIGNMENT;
    const int64_t es = io_size(desc->io_dtype);
    AliasCheck ac;
    ac.ins = {{x, nx * es}, {w, D * W * 4}, {b, b ? D * 4 : 0}, {state_in, state_in ? nst * 4 : 0}};
    ac.outs = {{y, nx * es}, {state_out, state_out ? nst * 4 : 0}};
    if (!ac.ok()) return SSM_ERR_ALIAS;
    ssm::ConvArgs a{};
    a.B = B; a.L = L; a.D = D; a.W = (int)W; a.silu = desc->fuse_silu; a.bf16 = desc->io_dtype == SSM_BF16;
    a.x = x; a.w = w; a.b = b; a.state_in = state_in; a.state_out = state_out; a.y = y;
    return hip_status(ssm::launch_conv1d(a, static_cast<hipStream_t>(stream)));
}

ssm_status ssm_scan_fwd_workspace_size(const ssm_scan_desc *desc, size_t *bytes) {
    ssm_status st = check_scan_desc(desc);
    if (st != SSM_OK) return st;
    if (!bytes) return SSM_ERR_NULL_ARG;
    *bytes = ssm::scan_fwd_workspace_bytes(desc->batch, desc->seqlen, desc->dim, desc->dstate,
                                           desc->conv_width, resolve_chunk(desc));
    return SSM_OK;
}

}  // extern "C"

namespace {

// ssm_scan_fwd, and with use_static its variant that takes the chunk
// summaries' buffer from the library's static scratch instead of `workspace`.
ssm_status scan_fwd_impl(const ssm_scan_desc *desc, const void *x, const void *dt_raw, const float *dt_bias,
                         const float *A_log, const void *B, const void *C, const float *Dskip, const void *z,
                         const float *conv_w, const float *conv_b, const float *conv_state_in,
                         float *conv_state_out, const float *h0, float *hT, void *y, void *workspace,
                         size_t workspace_bytes, void *stream, bool use_static) {
    ssm_status st = check_scan_desc(desc);
    if (st != SSM_OK) return st;
    const int64_t Bn = desc->batch, L = desc->seqlen, D = desc->dim, N = desc->dstate;
    const int W = desc->conv_width;
    const bool live = has_step_size(desc->disc);
    if (!live) dt_raw = nullptr, dt_bias = nullptr;   // not read
    if (!A_log || (L > 0 && (!x || (live && !dt_raw) || !B || !C || !y)) || (W > 0 && !conv_w))
        return SSM_ERR_NULL_ARG;
    for (const void *p : {(const void *)x, (const void *)dt_raw, (const void *)dt_bias, (const void *)A_log,
                          (const void *)B, (const void *)C, (const void *)Dskip, (const void *)z,
                          (const void *)conv_w, (const void *)conv_b, (const void *)conv_state_in,
                          (const void *)conv_state_out, (const void *)h0, (const void *)hT, (const void *)y,
                          (const void *)workspace})
        if (!aligned16(p)) return SSM_ERR_ALIGNMENT;
    const int64_t chunk = resolve_chunk(desc);
    {
        const int64_t K = cdiv(std::max<int64_t>(L, 1), chunk);   // chunks along time
        if (!grid_ok({Bn, cdiv(D, 16), K}) || !grid_ok({Bn, cdiv(D * N, 256)})) return SSM_ERR_BAD_SHAPE;
    }
    const size_t need = ssm::scan_fwd_workspace_bytes(Bn, L, D, N, W, chunk);
    if (use_static) {
        if (need > SSM_STATIC_SCRATCH_BYTES) return SSM_ERR_SCRATCH_LIMIT;
        workspace = nullptr;   // not part of the caller's buffers
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return SSM_ERR_WORKSPACE;
    }
    const int64_t es = io_size(desc->io_dtype);
    const int64_t nbld = Bn * L * D, nbln = Bn * L * N, nbdn = Bn * D * N, nst = Bn * (W > 0 ? W - 1 : 0) * D;
    AliasCheck ac;
    ac.ins = {{x, nbld * es},
              {dt_raw, dt_raw ? nbld * es : 0},
              {dt_bias, dt_bias ? D * 4 : 0},
              {A_log, D * N * 4},
              {B, nbln * es},
              {C, nbln * es},
              {Dskip, Dskip ? D * 4 : 0},
              {z, z ? nbld * es : 0},
              {conv_w, W > 0 ? D * W * 4 : 0},
              {conv_b, (W > 0 && conv_b) ? D * 4 : 0},
              {conv_state_in, (W > 0 && conv_state_in) ? nst * 4 : 0},
              {h0, h0 ? nbdn * 4 : 0}};
    ac.outs = {{y, nbld * es},
               {hT, hT ? nbdn * 4 : 0},
               {conv_state_out, (W > 0 && conv_state_out) ? nst * 4 : 0},
               {workspace, (need > 0 && workspace) ? (int64_t)need : 0}};
    ac.allowed = {{h0, hT}, {conv_state_in, conv_state_out}};
    if (!ac.ok()) return SSM_ERR_ALIAS;
    if (use_static && need > 0) {
        // this device's copy of the static buffer (first call: a symbol lookup)
        if (ssm::static_scratch(&workspace) != hipSuccess) return SSM_ERR_HIP;
    }
    ssm::ScanFwdArgs a{};
    a.B = Bn; a.L = L; a.D = D; a.N = N; a.W = W; a.bf16 = desc->io_dtype == SSM_BF16; a.disc = desc->disc;
    a.chunk_len = chunk;
    a.x = x; a.dt = dt_raw; a.dt_bias = dt_bias; a.A_log = A_log; a.Bm = B; a.Cm = C; a.Dskip = Dskip; a.z = z;
    a.conv_w = W > 0 ? conv_w : nullptr; a.conv_b = W > 0 ? conv_b : nullptr;
    a.conv_state_in = W > 0 ? conv_state_in : nullptr; a.conv_state_out = W > 0 ? conv_state_out : nullptr;
    a.h0 = h0; a.hT = hT; a.y = y; a.ws = workspace;
    return hip_status(ssm::launch_scan_fwd(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

ssm_status ssm_scan_fwd(const ssm_scan_desc *desc, const void *x, const void *dt_raw, const float *dt_bias,
                        const float *A_log, const void *B, const void *C, const float *Dskip, const void *z,
                        const float *conv_w, const float *conv_b, const float *conv_state_in,
                        float *conv_state_out, const float *h0, float *hT, void *y, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return scan_fwd_impl(desc, x, dt_raw, dt_bias, A_log, B, C, Dskip, z, conv_w, conv_b, conv_state_in,
                         conv_state_out, h0, hT, y, workspace, workspace_bytes, stream, false);
}

ssm_status ssm_scan_fwd_static(const ssm_scan_desc *desc, const void *x, const void *dt_raw,
                               const float *dt_bias, const float *A_log, const void *B, const void *C,
                               const float *Dskip, const void *z, const float *conv_w, const float *conv_b,
                               const float *conv_state_in, float *conv_state_out, const float *h0, float *hT,
                               void *y, void *stream) {
    return scan_fwd_impl(desc, x, dt_raw, dt_bias, A_log, B, C, Dskip, z, conv_w, conv_b, conv_state_in,
                         conv_state_out, h0, hT, y, nullptr, 0, stream, true);
}

ssm_status ssm_scan_bwd_workspace_size(const ssm_scan_desc *desc, size_t *bytes) {
    ssm_status st = check_scan_desc(desc);
    if (st != SSM_OK) return st;
    if (!bytes) return SSM_ERR_NULL_ARG;
    const int64_t chunk = ssm::scan_bwd_chunk(desc->batch, desc->seqlen, desc->dim, desc->dstate, desc->chunk_len);
    *bytes = ssm::scan_bwd_workspace_bytes(desc->batch, desc->seqlen, desc->dim, desc->dstate, chunk,
                                           desc->conv_width, io_size(desc->io_dtype));
    return SSM_OK;
}

ssm_status ssm_scan_bwd(const ssm_scan_desc *desc, const void *x, const void *dt_raw, const float *dt_bias,
                        const float *A_log, const void *B, const void *C, const float *Dskip, const void *z,
                        const float *conv_w, const float *conv_b, const float *conv_state_in, const float *h0,
                        const void *dy, const float *dhT, void *dx, void *d_dt_raw, float *d_dt_bias,
                        float *dA_log, void *dB, void *dC, float *dDskip, void *dz, float *dh0, float *dconv_w,
                        float *dconv_b, float *dconv_state_in, void *workspace, size_t workspace_bytes,
                        void *stream) {
    ssm_status st = check_scan_desc(desc);
    if (st != SSM_OK) return st;
    const int64_t Bn = desc->batch, L = desc->seqlen, D = desc->dim, N = desc->dstate;
    const int W = desc->conv_width;
    const bool live = has_step_size(desc->disc);
    if (!live) dt_raw = nullptr, dt_bias = nullptr, d_dt_raw = nullptr, d_dt_bias = nullptr;   // no step size
    if (!A_log || (L > 0 && (!x || (live && !dt_raw) || !B || !C || !dy)) || (W > 0 && !conv_w))
        return SSM_ERR_NULL_ARG;
    if (dz && !z) return SSM_ERR_NULL_ARG;
    if (W == 0 && (dconv_w || dconv_b || dconv_state_in)) return SSM_ERR_BAD_SHAPE;
    for (const void *p : {(const void *)x, (const void *)dt_raw, (const void *)dt_bias, (const void *)A_log,
                          (const void *)B, (const void *)C, (const void *)Dskip, (const void *)z,
                          (const void *)conv_w, (const void *)conv_b, (const void *)conv_state_in,
                          (const void *)h0, (const void *)dy, (const void *)dhT, (const void *)dx,
                          (const void *)d_dt_raw, (const void *)d_dt_bias, (const void *)dA_log,
                          (const void *)dB, (const void *)dC, (const void *)dDskip, (const void *)dz,
                          (const void *)dh0, (const void *)dconv_w, (const void *)dconv_b,
                          (const void *)dconv_state_in, (const void *)workspace})
        if (!aligned16(p)) return SSM_ERR_ALIGNMENT;
    const int64_t chunk = ssm::scan_bwd_chunk(Bn, L, D, N, desc->chunk_len);
    {
        const int64_t KC = cdiv(std::max<int64_t>(L, 1), chunk);   // chunks along time
        if (!grid_ok({Bn, cdiv(D, 48), KC}) || !grid_ok({Bn, cdiv(std::max<int64_t>(L, 1) * N, 256)}) ||
            !grid_ok({Bn, KC, cdiv(8 * D, 256)}) || !grid_ok({Bn, cdiv(D * N, 256)}) ||
            (W > 0 && !grid_ok({Bn, cdiv(cdiv(std::max<int64_t>(L, 1), 32) * D, 256)})) ||   // conv, conv backward
            // the sums' launch: dB, dC blocks then the parameter blocks
            cdiv(Bn * std::max<int64_t>(L, 1) * N, 256) + cdiv(std::max(D * N, D), 256) > kMaxGrid)
            return SSM_ERR_BAD_SHAPE;
    }
    const size_t need = ssm::scan_bwd_workspace_bytes(Bn, L, D, N, chunk, W, io_size(desc->io_dtype));
    if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE;
    const int64_t es = io_size(desc->io_dtype);
    const int64_t nbld = Bn * L * D, nbln = Bn * L * N, nbdn = Bn * D * N, nst = Bn * (W > 0 ? W - 1 : 0) * D;
    AliasCheck ac;
    ac.ins = {{x, nbld * es},
              {dt_raw, dt_raw ? nbld * es : 0},
              {dt_bias, dt_bias ? D * 4 : 0},
              {A_log, D * N * 4},
              {B, nbln * es},
              {C, nbln * es},
              {Dskip, Dskip ? D * 4 : 0},
              {z, z ? nbld * es : 0},
              {conv_w, W > 0 ? D * W * 4 : 0},
              {conv_b, (W > 0 && conv_b) ? D * 4 : 0},
              {conv_state_in, (W > 0 && conv_state_in) ? nst * 4 : 0},
              {h0, h0 ? nbdn * 4 : 0},
              {dy, nbld * es},
              {dhT, dhT ? nbdn * 4 : 0}};
    ac.outs = {{dx, dx ? nbld * es : 0},
               {d_dt_raw, d_dt_raw ? nbld * es : 0},
               {d_dt_bias, d_dt_bias ? D * 4 : 0},
               {dA_log, dA_log ? D * N * 4 : 0},
               {dB, dB ? nbln * es : 0},
               {dC, dC ? nbln * es : 0},
               {dDskip, dDskip ? D * 4 : 0},
               {dz, dz ? nbld * es : 0},
               {dh0, dh0 ? nbdn * 4 : 0},
               {dconv_w, dconv_w ? D * W * 4 : 0},
               {dconv_b, dconv_b ? D * 4 : 0},
               {dconv_state_in, dconv_state_in ? nst * 4 : 0},
               {workspace, (int64_t)need}};
    if (!ac.ok()) return SSM_ERR_ALIAS;
    ssm::ScanBwdArgs a{};
    a.B = Bn; a.L = L; a.D = D; a.N = N; a.W = W; a.bf16 = desc->io_dtype == SSM_BF16; a.disc = desc->disc;
    a.chunk = chunk;
    a.x = x; a.dt = dt_raw; a.dt_bias = dt_bias; a.A_log = A_log; a.Bm = B; a.Cm = C; a.Dskip = Dskip;
    a.z = z; a.h0 = h0; a.dy = dy; a.dhT = dhT;
    a.conv_w = W > 0 ? conv_w : nullptr; a.conv_b = W > 0 ? conv_b : nullptr;
    a.conv_state_in = W > 0 ? conv_state_in : nullptr;
    a.dx = dx; a.ddt = d_dt_raw; a.ddt_bias = d_dt_bias; a.dA_log = dA_log; a.dB = dB; a.dC = dC;
    a.dD = dDskip; a.dz = dz; a.dh0 = dh0;
    a.dconv_w = dconv_w; a.dconv_b = dconv_b; a.dconv_state_in = dconv_state_in; a.ws = workspace;
    return hip_status(ssm::launch_scan_bwd(a, static_cast<hipStream_t>(stream)));
}

ssm_status ssm_step(const ssm_step_desc *desc, void *h, float *conv_state, const void *x, const void *dt_raw,
                    const void *B, const void *C, const void *z, const float *conv_w, const float *conv_b,
                    const float *dt_bias, const float *A_log, const float *Dskip, void *y, void *stream) {
    if (!desc) return SSM_ERR_NULL_ARG;
    if (!valid_io(desc->io_dtype) || !valid_disc(desc->disc) || !valid_io(desc->state_dtype))
        return SSM_ERR_UNSUPPORTED;
    if (desc->nblocks < 1 || desc->nstreams < 1 || desc->dim < 1 || desc->dstate < 1 ||
        desc->dstate > SSM_MAX_DSTATE || desc->conv_width < 0 || desc->conv_width > SSM_MAX_CONV_WIDTH)
        return SSM_ERR_BAD_SHAPE;
    const int64_t K = desc->nblocks, S = desc->nstreams, D = desc->dim, N = desc->dstate;
    const int W = desc->conv_width;
    int64_t nh, nsd, nsn, nst;
    if (!elems({K, S, D, N}, &nh) || !elems({K, S, D}, &nsd) || !elems({K, S, N}, &nsn) ||
        !elems({K, S, (int64_t)(W > 0 ? W - 1 : 0), D}, &nst))
        return SSM_ERR_BAD_SHAPE;
    if (!grid_ok({K, S, cdiv(D * 16, 256)})) return SSM_ERR_BAD_SHAPE;
    const bool live = has_step_size(desc->disc);
    if (!live) dt_raw = nullptr, dt_bias = nullptr;   // not read
    if (!h || !x || (live && !dt_raw) || !B || !C || !A_log || !y || (W > 0 && !conv_w) ||
        (W > 1 && !conv_state))
        return SSM_ERR_NULL_ARG;
    for (const void *p : {(const void *)h, (const void *)conv_state, (const void *)x, (const void *)dt_raw,
                          (const void *)B, (const void *)C, (const void *)z, (const void *)conv_w,
                          (const void *)conv_b, (const void *)dt_bias, (const void *)A_log, (const void *)Dskip,
                          (const void *)y})
        if (!aligned16(p)) return SSM_ERR_ALIGNMENT;
    const int64_t es = io_size(desc->io_dtype);
    AliasCheck ac;
    ac.ins = {{x, nsd * es},
              {dt_raw, dt_raw ? nsd * es : 0},
              {B, nsn * es},
              {C, nsn * es},
              {z, z ? nsd * es : 0},
              {conv_w, W > 0 ? K * D * W * 4 : 0},
              {conv_b, (W > 0 && conv_b) ? K * D * 4 : 0},
              {dt_bias, dt_bias ? K * D * 4 : 0},
              {A_log, K * D * N * 4},
              {Dskip, Dskip ? K * D * 4 : 0}};
    ac.outs = {{h, nh * io_size(desc->state_dtype)}, {conv_state, W > 1 ? nst * 4 : 0}, {y, nsd * es}};
    if (!ac.ok()) return SSM_ERR_ALIAS;
    ssm::StepArgs a{};
    a.nblk = K; a.S = S; a.D = D; a.N = N; a.W = W; a.bf16 = desc->io_dtype == SSM_BF16; a.disc = desc->disc;
    a.state_bf16 = desc->state_dtype == SSM_BF16;
    a.h = h; a.conv_state = W > 1 ? conv_state : nullptr;
    a.x = x; a.dt = dt_raw; a.Bm = B; a.Cm = C; a.z = z;
    a.conv_w = W > 0 ? conv_w : nullptr; a.conv_b = W > 0 ? conv_b : nullptr;
    a.dt_bias = dt_bias; a.A_log = A_log; a.Dskip = Dskip; a.y = y;
    return hip_status(ssm::launch_step(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

ssm_status check_model_desc(const ssm_model_desc *d) {
    if (!d) return SSM_ERR_NULL_ARG;
    if (d->reserved != 0) return SSM_ERR_UNSUPPORTED;
    if (d->nstreams < 1 || d->vocab < 1 || d->d_model < 1 || d->d_model > SSM_MAX_D_MODEL || d->n_layers < 1 ||
        d->d_inner < 1 || d->d_state < 1 || d->d_state > SSM_MAX_DSTATE || d->dt_rank < 1 ||
        d->conv_width < 1 || d->conv_width > SSM_MAX_CONV_WIDTH)
        return SSM_ERR_BAD_SHAPE;
    int64_t n;
    const int64_t S = d->nstreams, Di = d->d_inner;
    if (!elems({S, d->vocab}, &n) || !elems({d->n_layers, S, Di, d->d_state}, &n) ||
        !elems({d->n_layers, S, d->conv_width - 1, Di}, &n) || !elems({S, 2 * Di}, &n) ||
        !elems({(int64_t)d->vocab, d->d_model}, &n) || !elems({2 * Di, d->d_model}, &n) ||
        !elems({(int64_t)d->dt_rank + 2 * d->d_state, Di}, &n))
        return SSM_ERR_BAD_SHAPE;
    const int64_t widest = std::max<int64_t>({2 * Di, (int64_t)d->vocab, (int64_t)d->d_model,
                                              (int64_t)d->dt_rank + 2 * d->d_state});
    if (!grid_ok({cdiv(S, 16), cdiv(widest, 16)}) || !grid_ok({S, cdiv(Di * 16, 256)})) return SSM_ERR_BAD_SHAPE;
    return SSM_OK;
}

}  // namespace

extern "C" {

ssm_status ssm_model_decode_workspace_size(const ssm_model_desc *desc, size_t *bytes) {
    ssm_status st = check_model_desc(desc);
    if (st != SSM_OK) return st;
    if (!bytes) return SSM_ERR_NULL_ARG;
    *bytes = ssm::model_workspace_bytes(desc->nstreams, desc->d_model, desc->d_inner, desc->d_state,
                                        desc->dt_rank);
    return SSM_OK;
}

ssm_status ssm_model_decode_step(const ssm_model_desc *desc, const float *emb, const float *norm_f_w,
                                 const float *norm_f_b, const ssm_layer_weights *layers,
                                 const int32_t *tokens, float *h, float *conv_state, float *logits,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    ssm_status st = check_model_desc(desc);
    if (st != SSM_OK) return st;
    const int64_t S = desc->nstreams, V = desc->vocab, dm = desc->d_model, nl = desc->n_layers;
    const int64_t Di = desc->d_inner, N = desc->d_state, R = desc->dt_rank, W = desc->conv_width;
    if (!emb || !layers || !tokens || !h || !logits || (W > 1 && !conv_state)) return SSM_ERR_NULL_ARG;
    for (int64_t l = 0; l < nl; ++l) {
        const ssm_layer_weights &L = layers[l];
        if (!L.in_proj || !L.conv_w || !L.x_proj || !L.dt_proj_w || !L.A_log || !L.out_proj)
            return SSM_ERR_NULL_ARG;
    }
    const size_t need = ssm::model_workspace_bytes(S, dm, Di, N, R);
    if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE;
    AliasCheck ac;
    ac.ins = {{emb, V * dm * 4}, {norm_f_w, norm_f_w ? dm * 4 : 0}, {norm_f_b, norm_f_b ? dm * 4 : 0},
              {tokens, S * 4}};
    for (int64_t l = 0; l < nl; ++l) {
        const ssm_layer_weights &L = layers[l];
        const std::vector<Range> r = {{L.norm_w, L.norm_w ? dm * 4 : 0}, {L.norm_b, L.norm_b ? dm * 4 : 0},
                                      {L.in_proj, 2 * Di * dm * 4},   {L.conv_w, Di * W * 4},
                                      {L.conv_b, L.conv_b ? Di * 4 : 0}, {L.x_proj, (R + 2 * N) * Di * 4},
                                      {L.dt_proj_w, Di * R * 4},      {L.dt_proj_b, L.dt_proj_b ? Di * 4 : 0},
                                      {L.A_log, Di * N * 4},          {L.Dskip, L.Dskip ? Di * 4 : 0},
                                      {L.out_proj, dm * Di * 4}};
        for (const Range &x : r) {
            if (!aligned16(x.p)) return SSM_ERR_ALIGNMENT;
            ac.ins.push_back(x);
        }
    }
    for (const void *p : {(const void *)emb, (const void *)norm_f_w, (const void *)norm_f_b, (const void *)h,
                          (const void *)conv_state, (const void *)logits, (const void *)workspace})
        if (!aligned16(p)) return SSM_ERR_ALIGNMENT;
    // token ids are read one by one: 4-byte alignment, so that step t of a
    // [T, S] token buffer can be passed as is
    if ((reinterpret_cast<uintptr_t>(tokens) & 3u) != 0) return SSM_ERR_ALIGNMENT;
    ac.outs = {{h, nl * S * Di * N * 4},
               {conv_state, W > 1 ? nl * S * (W - 1) * Di * 4 : 0},
               {logits, S * V * 4},
               {workspace, (int64_t)need}};
    if (!ac.ok()) return SSM_ERR_ALIAS;
    std::vector<ssm::ModelLayer> ls((size_t)nl);
    for (int64_t l = 0; l < nl; ++l) {
        const ssm_layer_weights &L = layers[l];
        ls[(size_t)l] = ssm::ModelLayer{L.norm_w, L.norm_b, L.in_proj, L.conv_w, L.conv_b, L.x_proj,
                                        L.dt_proj_w, L.dt_proj_b, L.A_log, L.Dskip, L.out_proj};
    }
    ssm::ModelArgs a{};
    a.S = S; a.V = (int)V; a.dm = (int)dm; a.nl = (int)nl; a.Di = (int)Di; a.N = (int)N; a.R = (int)R; a.W = (int)W;
    a.emb = emb; a.norm_f_w = norm_f_w; a.norm_f_b = norm_f_b; a.layers = ls.data(); a.tok = tokens;
    a.h = h; a.conv = W > 1 ? conv_state : nullptr; a.logits = logits; a.ws = workspace;
    return hip_status(ssm::launch_model_decode(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
