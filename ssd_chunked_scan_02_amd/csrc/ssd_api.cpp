// C ABI of libssd (declared in include/ssd.h): argument validation, workspace sizing and
// dispatch to the kernels.  Every check runs before the first HIP call.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include "ssd_bwd_launch.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_chunk(int chunk) {
    return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128 || chunk == 256;
}

// Shape checks shared by forward and step.  Returns SSD_OK or an error code.
int check_dims(const ssd_dims* d, bool forward) {
    if (!d) return SSD_ERR_INVALID;
    if (d->batch < 0 || d->nheads < 1 || d->ngroups < 1 || d->headdim < 1 || d->dstate < 1)
        return SSD_ERR_INVALID;
    if (forward && d->seqlen < 0) return SSD_ERR_INVALID;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_INVALID;
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16) return SSD_ERR_INVALID;
    if (d->decay != SSD_DECAY_SCALAR && d->decay != SSD_DECAY_DIAG) return SSD_ERR_INVALID;
    if (d->batch > kMaxElems || d->nheads > kMaxElems || d->headdim > 4096 || d->dstate > 4096)
        return SSD_ERR_INVALID;
    const int64_t T = forward ? d->seqlen : 1;
    if (T > kMaxElems) return SSD_ERR_INVALID;
    // element counts of the largest tensors must stay well inside int64
    const double big = (double)d->batch * (double)(T > 0 ? T : 1) * (double)d->nheads *
                       (double)(d->headdim > d->dstate ? d->headdim : d->dstate);
    if (big > (double)kMaxElems * 1024.0) return SSD_ERR_INVALID;
    if (!forward || d->decay == SSD_DECAY_SCALAR) {
        if (!ssd::shape_supported(d->dtype, (int)d->dstate, (int)d->headdim)) return SSD_ERR_UNSUPPORTED;
    }
    return SSD_OK;
}

// (varlen: a packed variable-length batch of d->batch sequences of at most d->seqlen tokens)
size_t workspace_needed(const ssd_dims* d, int chunk, bool varlen = false) {
    if (d->seqlen == 0 || d->batch == 0) return 0;
    const int64_t nchunks = (d->seqlen + chunk - 1) / chunk;
    if (d->decay == SSD_DECAY_DIAG)
        return ssd::diag_workspace_bytes(d->dtype, d->batch, d->nheads, d->seqlen, (int)d->dstate, (int)d->headdim,
                                         chunk, varlen);
    if (ssd::fast_path_applies(d->dtype, d->decay, (int)d->dstate, (int)d->headdim, chunk, d->nheads, d->ngroups))
        return ssd::fast_workspace_bytes(d->batch, d->nheads, d->ngroups, d->seqlen, (int)d->dstate, chunk, false,
                                         varlen);
    return ssd::scores_bytes(d->batch, d->ngroups, nchunks, chunk);
}

// Workspace of ssd_forward_dt: the fused paths need what ssd_forward needs (plus log2 of the
// input scale on the scalar fast path); the generic composition adds log a and the scaled input
// (for a packed batch, rows for batch * seqlen tokens, which bound its token count).
size_t workspace_needed_dt(const ssd_dims* d, int chunk, bool scale_input, bool varlen = false) {
    if (d->seqlen == 0 || d->batch == 0) return 0;
    const int N = (int)d->dstate, P = (int)d->headdim;
    if (ssd::discretization_fused(d->dtype, d->decay, N, P, chunk, d->nheads, d->ngroups)) {
        if (d->decay == SSD_DECAY_DIAG)
            return ssd::diag_workspace_bytes(d->dtype, d->batch, d->nheads, d->seqlen, N, P, chunk, varlen);
        return ssd::fast_workspace_bytes(d->batch, d->nheads, d->ngroups, d->seqlen, N, chunk, scale_input, varlen);
    }
    const size_t own = ssd::generic_workspace_bytes(d->dtype, d->decay, d->batch, d->nheads, d->ngroups,
                                                    d->seqlen, N, P, chunk);
    return ssd::dt_generic_layout(own, d->batch, d->seqlen, d->nheads, d->decay == SSD_DECAY_DIAG ? N : 1, P,
                                  d->dtype == SSD_BF16 ? 2 : 4, scale_input)
        .total;
}

int check_forward(const ssd_dims* d, int chunk) {
    int rc = check_dims(d, true);
    if (rc != SSD_OK) return rc;
    if (!valid_chunk(chunk)) return SSD_ERR_UNSUPPORTED;
    if (d->decay == SSD_DECAY_DIAG) {
        const size_t lds = ssd::diag_lds_bytes(d->dtype, (int)d->dstate, (int)d->headdim, chunk);
        if (lds == 0 || lds > ssd::kMaxLds) return SSD_ERR_UNSUPPORTED;
        return SSD_OK;
    }
    if (ssd::walk_lds_bytes(d->dtype, (int)d->dstate, (int)d->headdim, chunk) > ssd::kMaxLds)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Backward pass: scalar decay with N in {16, 32, 64, 128}, or diagonal decay with N in {16, 32,
// 64}; P in {16, 32, 64}; either dtype.
int check_backward(const ssd_dims* d) {
    int rc = check_dims(d, true);
    if (rc != SSD_OK) return rc;
    if (!ssd::backward_shape_supported((int)d->dstate, (int)d->headdim, d->decay)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

struct Discretization {
    const float* dt;
    const float* dt_bias;
    const float* A_log;
    bool scale_input;
};

// A packed variable-length batch: sequence offsets on the device and the packed token count.
struct Varlen {
    const int64_t* cu_seqlens;
    int64_t total;
};

// ssd_forward (disc null: log_a given), ssd_forward_dt (disc set: log_a null), and their packed
// variable-length forms (vl set).
int forward_impl(const ssd_dims* d, const void* x, const float* log_a, const Discretization* disc,
                 const void* B, const void* C, const float* D, int chunk, const float* init_state,
                 void* y, float* final_state, void* workspace, size_t workspace_bytes, void* stream,
                 void* const* events, int n_events, int* n_launches, const Varlen* vl = nullptr,
                 bool check_only = false) {
    if (n_launches) *n_launches = 0;
    if (events && n_events < 2 * SSD_MAX_LAUNCHES) return SSD_ERR_INVALID;
    int rc = check_forward(d, chunk);
    if (rc != SSD_OK) return rc;
    if (vl) {
        // (every sequence has at most seqlen tokens, so the packed axis has at most batch * seqlen)
        if (vl->total < 0 || vl->total > kMaxElems || vl->total > d->batch * d->seqlen) return SSD_ERR_INVALID;
        if (d->batch > 0 && (!vl->cu_seqlens || ((uintptr_t)vl->cu_seqlens & 7u) != 0)) return SSD_ERR_INVALID;
        // (every packed tensor's element count must stay well inside int64, as for the batched form)
        if ((double)vl->total * (double)d->nheads * (double)(d->headdim > d->dstate ? d->headdim : d->dstate) >
            (double)kMaxElems * 1024.0)
            return SSD_ERR_INVALID;
    }
    const bool has_tokens = d->batch > 0 && d->seqlen > 0 && (!vl || vl->total > 0);
    const float* decay_in = disc ? disc->dt : log_a;
    if (has_tokens && (!x || !decay_in || !B || !C || !y)) return SSD_ERR_INVALID;
    if (has_tokens && disc && !disc->A_log) return SSD_ERR_INVALID;
    const void* ptrs[] = {x, log_a, B, C, D, init_state, y, final_state, workspace,
                          disc ? disc->dt : nullptr, disc ? disc->dt_bias : nullptr, disc ? disc->A_log : nullptr};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    const size_t need = disc ? workspace_needed_dt(d, chunk, disc->scale_input, vl != nullptr)
                             : workspace_needed(d, chunk, vl != nullptr);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_INVALID;
    if (check_only || d->batch == 0) return SSD_OK;
    if ((d->seqlen == 0 || (vl && vl->total == 0)) && !final_state) return SSD_OK;

    int count = 0;
    ssd::ForwardLaunch fl{};
    fl.dtype = d->dtype;
    fl.decay = d->decay;
    fl.batch = d->batch;
    fl.seqlen = d->seqlen;
    fl.nheads = d->nheads;
    fl.ngroups = d->ngroups;
    fl.headdim = d->headdim;
    fl.dstate = d->dstate;
    fl.chunk = chunk;
    fl.nchunks = (int)((d->seqlen + chunk - 1) / chunk);
    fl.x = x;
    fl.log_a = log_a;
    if (disc) {
        fl.dt = disc->dt;
        fl.dt_bias = disc->dt_bias;
        fl.A_log = disc->A_log;
        fl.scale_input = disc->scale_input ? 1 : 0;
    }
    fl.Bm = B;
    fl.Cm = C;
    fl.D = D;
    fl.init = init_state;
    fl.y = y;
    fl.final_state = final_state;
    fl.scores = static_cast<float*>(workspace);
    fl.events = reinterpret_cast<hipEvent_t const*>(events);
    fl.n_events = events ? n_events : 0;
    fl.n_launches = &count;
    fl.first_launch = 0;
    if (vl) {
        fl.seq_off = vl->cu_seqlens;
        fl.total = vl->total;
        // (no tokens at all: every sequence is empty, its final state its initial state)
        if (vl->total == 0) fl.seqlen = 0;
    }
    rc = ssd::launch_forward(fl, static_cast<hipStream_t>(stream));
    if (n_launches) *n_launches = count;
    if (rc == -2) return SSD_ERR_UNSUPPORTED;
    return rc == 0 ? SSD_OK : SSD_ERR_HIP;
}

// ssd_step (disc null) and ssd_step_dt.
int step_impl(const ssd_dims* d, float* state, const void* x_t, const float* log_a_t, const Discretization* disc,
              const void* B_t, const void* C_t, const float* D, void* y_t, void* stream) {
    int rc = check_dims(d, false);
    if (rc != SSD_OK) return rc;
    if (d->headdim > 256 || 256 % d->headdim != 0) return SSD_ERR_UNSUPPORTED;
    if (d->batch == 0) return SSD_OK;
    const float* decay_in = disc ? disc->dt : log_a_t;
    if (!state || !x_t || !decay_in || !B_t || !C_t || !y_t || (disc && !disc->A_log)) return SSD_ERR_INVALID;
    const void* ptrs[] = {state, x_t, log_a_t, B_t, C_t, D, y_t,
                          disc ? disc->dt : nullptr, disc ? disc->dt_bias : nullptr, disc ? disc->A_log : nullptr};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::StepParams sp{state, x_t, log_a_t, B_t, C_t, D, y_t, d->nheads, d->ngroups,
                       (int)d->headdim, (int)d->dstate, d->decay == SSD_DECAY_DIAG ? 1 : 0};
    if (disc) {
        sp.dt_t = disc->dt;
        sp.dt_bias = disc->dt_bias;
        sp.A_log = disc->A_log;
        sp.scale_input = disc->scale_input ? 1 : 0;
    }
    rc = ssd::launch_step(sp, d->dtype, d->batch * d->nheads, static_cast<hipStream_t>(stream));
    return rc == 0 ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

extern "C" {

size_t ssd_forward_varlen_workspace_bytes(const ssd_dims* dims, int chunk) {
    if (check_forward(dims, chunk) != SSD_OK) return 0;
    return workspace_needed(dims, chunk, true);
}

int ssd_forward_varlen(const ssd_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens, const void* x,
                       const float* log_a, const void* B, const void* C, const float* D, int chunk,
                       const float* init_state, void* y, float* final_state, void* workspace, size_t workspace_bytes,
                       void* stream, void* const* events, int n_events, int* n_launches) {
    const Varlen vl{cu_seqlens, total_tokens};
    return forward_impl(dims, x, log_a, nullptr, B, C, D, chunk, init_state, y, final_state, workspace,
                        workspace_bytes, stream, events, n_events, n_launches, &vl);
}

size_t ssd_forward_dt_varlen_workspace_bytes(const ssd_dims* dims, int chunk, int scale_input) {
    if (check_forward(dims, chunk) != SSD_OK) return 0;
    return workspace_needed_dt(dims, chunk, scale_input != 0, true);
}

int ssd_forward_dt_varlen(const ssd_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens, const void* x,
                          const float* dt, const float* dt_bias, const float* A_log, int scale_input, const void* B,
                          const void* C, const float* D, int chunk, const float* init_state, void* y,
                          float* final_state, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events, int n_events, int* n_launches) {
    const Varlen vl{cu_seqlens, total_tokens};
    const Discretization disc{dt, dt_bias, A_log, scale_input != 0};
    return forward_impl(dims, x, nullptr, &disc, B, C, D, chunk, init_state, y, final_state, workspace,
                        workspace_bytes, stream, events, n_events, n_launches, &vl);
}

size_t ssd_forward_workspace_bytes(const ssd_dims* dims, int chunk) {
    if (check_forward(dims, chunk) != SSD_OK) return 0;
    return workspace_needed(dims, chunk);
}

int ssd_forward(const ssd_dims* d, const void* x, const float* log_a, const void* B, const void* C,
                const float* D, int chunk, const float* init_state, void* y, float* final_state,
                void* workspace, size_t workspace_bytes, void* stream) {
    return ssd_forward_profiled(d, x, log_a, B, C, D, chunk, init_state, y, final_state, workspace,
                                workspace_bytes, stream, nullptr, 0, nullptr);
}

int ssd_forward_profiled(const ssd_dims* d, const void* x, const float* log_a, const void* B,
                         const void* C, const float* D, int chunk, const float* init_state,
                         void* y, float* final_state, void* workspace, size_t workspace_bytes,
                         void* stream, void* const* events, int n_events, int* n_launches) {
    return forward_impl(d, x, log_a, nullptr, B, C, D, chunk, init_state, y, final_state, workspace,
                        workspace_bytes, stream, events, n_events, n_launches);
}

size_t ssd_forward_dt_workspace_bytes(const ssd_dims* dims, int chunk, int scale_input) {
    if (check_forward(dims, chunk) != SSD_OK) return 0;
    return workspace_needed_dt(dims, chunk, scale_input != 0);
}

int ssd_forward_dt(const ssd_dims* d, const void* x, const float* dt, const float* dt_bias,
                   const float* A_log, int scale_input, const void* B, const void* C,
                   const float* D, int chunk, const float* init_state, void* y,
                   float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    return ssd_forward_dt_profiled(d, x, dt, dt_bias, A_log, scale_input, B, C, D, chunk, init_state, y,
                                   final_state, workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

int ssd_forward_dt_profiled(const ssd_dims* d, const void* x, const float* dt,
                            const float* dt_bias, const float* A_log, int scale_input,
                            const void* B, const void* C, const float* D, int chunk,
                            const float* init_state, void* y, float* final_state,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events, int n_events, int* n_launches) {
    const Discretization disc{dt, dt_bias, A_log, scale_input != 0};
    return forward_impl(d, x, nullptr, &disc, B, C, D, chunk, init_state, y, final_state, workspace,
                        workspace_bytes, stream, events, n_events, n_launches);
}

int ssd_step(const ssd_dims* d, float* state, const void* x_t, const float* log_a_t, const void* B_t,
             const void* C_t, const float* D, void* y_t, void* stream) {
    return step_impl(d, state, x_t, log_a_t, nullptr, B_t, C_t, D, y_t, stream);
}

int ssd_step_dt(const ssd_dims* d, float* state, const void* x_t, const float* dt_t,
                const float* dt_bias, const float* A_log, int scale_input, const void* B_t,
                const void* C_t, const float* D, void* y_t, void* stream) {
    const Discretization disc{dt_t, dt_bias, A_log, scale_input != 0};
    return step_impl(d, state, x_t, nullptr, &disc, B_t, C_t, D, y_t, stream);
}

size_t ssd_backward_workspace_bytes(const ssd_dims* d) {
    if (check_backward(d) != SSD_OK || d->batch == 0) return 0;
    return ssd::backward_workspace_bytes(d->batch, d->nheads, d->seqlen, (int)d->dstate, (int)d->headdim, d->decay);
}

int ssd_backward(const ssd_dims* d, const void* x, const float* log_a, const void* B, const void* C,
                 const float* D, const float* init_state, const void* dy, const float* dfinal, void* dx,
                 float* dlog_a, float* dB, float* dC, float* dD, float* dinit, void* workspace,
                 size_t workspace_bytes, void* stream) {
    return ssd_backward_profiled(d, x, log_a, B, C, D, init_state, dy, dfinal, dx, dlog_a, dB, dC, dD, dinit,
                                 workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

}  // extern "C"

namespace {

// ssd_backward(_profiled) (vl null) and ssd_backward_varlen (vl set).
int backward_impl(const ssd_dims* d, const void* x, const float* log_a, const void* B, const void* C, const float* D,
                  const float* init_state, const void* dy, const float* dfinal, void* dx, float* dlog_a, float* dB,
                  float* dC, float* dD, float* dinit, void* workspace, size_t workspace_bytes, void* stream,
                  void* const* events, int n_events, int* n_launches, const Varlen* vl) {
    if (n_launches) *n_launches = 0;
    if (events && n_events < 2 * SSD_MAX_LAUNCHES) return SSD_ERR_INVALID;
    int rc = check_backward(d);
    if (rc != SSD_OK) return rc;
    if (vl) {
        if (vl->total < 0 || vl->total > d->batch * d->seqlen) return SSD_ERR_INVALID;
        if (d->batch > 0 && (!vl->cu_seqlens || ((uintptr_t)vl->cu_seqlens & 7u) != 0)) return SSD_ERR_INVALID;
    }
    const bool has_tokens = d->batch > 0 && d->seqlen > 0 && (!vl || vl->total > 0);
    if (has_tokens && (!x || !log_a || !B || !C || !dy || !dx || !dlog_a || !dB || !dC)) return SSD_ERR_INVALID;
    const void* ptrs[] = {x, log_a, B, C, D, init_state, dy, dfinal, dx, dlog_a, dB, dC, dD, dinit, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    const size_t need = ssd_backward_workspace_bytes(d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_INVALID;
    if (d->batch == 0 && !dD) return SSD_OK;
    ssd::BackwardLaunch bl{};
    bl.dtype = d->dtype;
    bl.decay = d->decay;
    bl.headdim = d->headdim;
    bl.dstate = d->dstate;
    ssd::BwdParams& p = bl.p;
    p.x = x;
    p.log_a = log_a;
    p.Bm = B;
    p.Cm = C;
    p.D = D;
    p.init = init_state;
    p.dy = dy;
    p.dfinal = dfinal;
    p.dx = dx;
    p.dlog_a = dlog_a;
    p.dB = dB;
    p.dC = dC;
    p.dD = dD;
    p.dinit = dinit;
    p.batch = d->batch;
    p.seqlen = d->seqlen;
    p.nheads = d->nheads;
    p.ngroups = d->ngroups;
    p.nchunks = (int)((d->seqlen + ssd::backward_chunk() - 1) / ssd::backward_chunk());
    ssd::bind_backward_workspace(p, workspace, (int)d->dstate, (int)d->headdim, d->decay);
    if (vl) {
        p.seq_off = vl->cu_seqlens;
        p.total = vl->total;
    }
    int count = 0;
    bl.events = reinterpret_cast<hipEvent_t const*>(events);
    bl.n_events = events ? n_events : 0;
    bl.n_launches = &count;
    rc = ssd::launch_backward(bl, static_cast<hipStream_t>(stream));
    if (n_launches) *n_launches = count;
    if (rc == -2) return SSD_ERR_UNSUPPORTED;
    return rc == 0 ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

extern "C" {

int ssd_backward_profiled(const ssd_dims* d, const void* x, const float* log_a, const void* B, const void* C,
                          const float* D, const float* init_state, const void* dy, const float* dfinal, void* dx,
                          float* dlog_a, float* dB, float* dC, float* dD, float* dinit, void* workspace,
                          size_t workspace_bytes, void* stream, void* const* events, int n_events, int* n_launches) {
    return backward_impl(d, x, log_a, B, C, D, init_state, dy, dfinal, dx, dlog_a, dB, dC, dD, dinit, workspace,
                         workspace_bytes, stream, events, n_events, n_launches, nullptr);
}

size_t ssd_backward_varlen_workspace_bytes(const ssd_dims* d) { return ssd_backward_workspace_bytes(d); }

int ssd_backward_varlen(const ssd_dims* d, const int64_t* cu_seqlens, int64_t total_tokens, const void* x,
                        const float* log_a, const void* B, const void* C, const float* D, const float* init_state,
                        const void* dy, const float* dfinal, void* dx, float* dlog_a, float* dB, float* dC, float* dD,
                        float* dinit, void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                        int n_events, int* n_launches) {
    const Varlen vl{cu_seqlens, total_tokens};
    return backward_impl(d, x, log_a, B, C, D, init_state, dy, dfinal, dx, dlog_a, dB, dC, dD, dinit, workspace,
                         workspace_bytes, stream, events, n_events, n_launches, &vl);
}

size_t ssd_backward_dt_workspace_bytes(const ssd_dims* d, int scale_input) {
    if (check_backward(d) != SSD_OK || d->batch == 0) return 0;
    return ssd::dt_backward_layout(d->batch, d->nheads, d->seqlen, (int)d->dstate, (int)d->headdim,
                                   d->dtype == SSD_BF16 ? 2 : 4, scale_input != 0, d->decay)
        .total;
}

}  // extern "C"

namespace {

// ssd_backward_dt (vl null) and ssd_backward_dt_varlen (vl set).
int backward_dt_impl(const ssd_dims* d, const void* x, const float* dt, const float* dt_bias, const float* A_log,
                     int scale_input, const void* B, const void* C, const float* D, const float* init_state,
                     const void* dy, const float* dfinal, void* dx, float* ddt, float* dA_log, float* ddt_bias,
                     float* dB, float* dC, float* dD, float* dinit, void* workspace, size_t workspace_bytes,
                     void* stream, const Varlen* vl) {
    int rc = check_backward(d);
    if (rc != SSD_OK) return rc;
    if (vl) {
        if (vl->total < 0 || vl->total > d->batch * d->seqlen) return SSD_ERR_INVALID;
        if (d->batch > 0 && (!vl->cu_seqlens || ((uintptr_t)vl->cu_seqlens & 7u) != 0)) return SSD_ERR_INVALID;
    }
    const bool has_tokens = d->batch > 0 && d->seqlen > 0 && (!vl || vl->total > 0);
    if (has_tokens && (!x || !dt || !A_log || !B || !C || !dy || !dx || !ddt || !dB || !dC)) return SSD_ERR_INVALID;
    if (!A_log && (dA_log || ddt_bias)) return SSD_ERR_INVALID;
    const void* ptrs[] = {x, dt, dt_bias, A_log, B, C, D, init_state, dy, dfinal, dx, ddt, dA_log, ddt_bias,
                          dB, dC, dD, dinit, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    const size_t need = ssd_backward_dt_workspace_bytes(d, scale_input);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_INVALID;
    ssd::BackwardLaunch bl{};
    bl.dtype = d->dtype;
    bl.decay = d->decay;
    bl.headdim = d->headdim;
    bl.dstate = d->dstate;
    ssd::BwdParams& p = bl.p;
    p.Bm = B;
    p.Cm = C;
    p.init = init_state;
    p.dy = dy;
    p.dfinal = dfinal;
    p.dB = dB;
    p.dC = dC;
    p.dinit = dinit;
    p.batch = d->batch;
    p.seqlen = d->seqlen;
    p.nheads = d->nheads;
    p.ngroups = d->ngroups;
    p.nchunks = (int)((d->seqlen + ssd::backward_chunk() - 1) / ssd::backward_chunk());
    if (vl) {
        p.seq_off = vl->cu_seqlens;
        p.total = vl->total;
    }
    int count = 0;
    bl.n_launches = &count;
    ssd::DtBackwardArgs a{x, dt, dt_bias, A_log, scale_input != 0, D, dy, dx, ddt, dA_log, ddt_bias, dD, workspace};
    rc = ssd::launch_backward_dt(bl, a, static_cast<hipStream_t>(stream));
    if (rc == -2) return SSD_ERR_UNSUPPORTED;
    return rc == 0 ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

extern "C" {

int ssd_backward_dt(const ssd_dims* d, const void* x, const float* dt, const float* dt_bias, const float* A_log,
                    int scale_input, const void* B, const void* C, const float* D, const float* init_state,
                    const void* dy, const float* dfinal, void* dx, float* ddt, float* dA_log, float* ddt_bias,
                    float* dB, float* dC, float* dD, float* dinit, void* workspace, size_t workspace_bytes,
                    void* stream) {
    return backward_dt_impl(d, x, dt, dt_bias, A_log, scale_input, B, C, D, init_state, dy, dfinal, dx, ddt, dA_log,
                            ddt_bias, dB, dC, dD, dinit, workspace, workspace_bytes, stream, nullptr);
}

size_t ssd_backward_dt_varlen_workspace_bytes(const ssd_dims* d, int scale_input) {
    return ssd_backward_dt_workspace_bytes(d, scale_input);
}

int ssd_backward_dt_varlen(const ssd_dims* d, const int64_t* cu_seqlens, int64_t total_tokens, const void* x,
                           const float* dt, const float* dt_bias, const float* A_log, int scale_input, const void* B,
                           const void* C, const float* D, const float* init_state, const void* dy,
                           const float* dfinal, void* dx, float* ddt, float* dA_log, float* ddt_bias, float* dB,
                           float* dC, float* dD, float* dinit, void* workspace, size_t workspace_bytes,
                           void* stream) {
    const Varlen vl{cu_seqlens, total_tokens};
    return backward_dt_impl(d, x, dt, dt_bias, A_log, scale_input, B, C, D, init_state, dy, dfinal, dx, ddt, dA_log,
                            ddt_bias, dB, dC, dD, dinit, workspace, workspace_bytes, stream, &vl);
}

size_t ssd_noalloc_scratch_bytes(void) { return ssd::noalloc_scratch_bytes(); }

int ssd_forward_noalloc(const ssd_dims* d, const void* x, const float* log_a, const void* B, const void* C,
                        const float* D, int chunk, const float* init_state, void* y, float* final_state,
                        void* stream) {
    // every check first (the workspace stands in as the scratch array's size at a dummy aligned
    // address), then the one HIP call that finds this device's copy of the array
    int rc = check_forward(d, chunk);
    if (rc != SSD_OK) return rc;
    const size_t need = workspace_needed(d, chunk);
    if (need > ssd::noalloc_scratch_bytes()) return SSD_ERR_SCRATCH;
    alignas(256) static const unsigned char probe[16] = {};
    rc = forward_impl(d, x, log_a, nullptr, B, C, D, chunk, init_state, y, final_state, (void*)probe,
                      ssd::noalloc_scratch_bytes(), stream, nullptr, 0, nullptr, nullptr, true);
    if (rc != SSD_OK) return rc;
    if (d->batch == 0) return SSD_OK;
    void* ws = nullptr;
    if (need > 0) {
        int hip_rc = 0;
        ws = ssd::noalloc_scratch(&hip_rc);
        if (!ws) return SSD_ERR_HIP;
    }
    return forward_impl(d, x, log_a, nullptr, B, C, D, chunk, init_state, y, final_state, ws, need, stream,
                        nullptr, 0, nullptr);
}

const char* ssd_strerror(int code) {
    switch (code) {
        case SSD_OK: return "success";
        case SSD_ERR_INVALID: return "invalid argument (null pointer, bad dimension or workspace too small)";
        case SSD_ERR_UNSUPPORTED: return "unsupported configuration (chunk, dstate, headdim, dtype or decay kind)";
        case SSD_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case SSD_ERR_HIP: return "HIP runtime rejected a kernel launch";
        case SSD_ERR_SCRATCH:
            return "the call needs more workspace than ssd_forward_noalloc's fixed scratch array holds "
                   "(ssd_noalloc_scratch_bytes); call ssd_forward with a workspace instead";
        default: return "unknown error code";
    }
}

}  // extern "C"
