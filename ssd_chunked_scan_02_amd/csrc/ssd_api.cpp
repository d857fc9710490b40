// C ABI of libssd (declared in include/ssd.h): argument validation, workspace sizing and
// dispatch to the kernels.  Every check runs before the first HIP call.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include "ssd_launch.h"

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

size_t workspace_needed(const ssd_dims* d, int chunk) {
    if (d->seqlen == 0 || d->batch == 0) return 0;
    const int64_t nchunks = (d->seqlen + chunk - 1) / chunk;
    if (d->decay == SSD_DECAY_DIAG)
        return ssd::diag_workspace_bytes(d->dtype, d->batch, d->nheads, d->seqlen, (int)d->dstate, (int)d->headdim,
                                         chunk);
    if (ssd::fast_path_applies(d->dtype, d->decay, (int)d->dstate, (int)d->headdim, chunk, d->nheads, d->ngroups))
        return ssd::fast_workspace_bytes(d->batch, d->nheads, d->ngroups, d->seqlen, (int)d->dstate, chunk);
    return ssd::scores_bytes(d->batch, d->ngroups, nchunks, chunk);
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

}  // namespace

extern "C" {

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
    if (n_launches) *n_launches = 0;
    if (events && n_events < 2 * SSD_MAX_LAUNCHES) return SSD_ERR_INVALID;
    int rc = check_forward(d, chunk);
    if (rc != SSD_OK) return rc;
    const bool has_tokens = d->batch > 0 && d->seqlen > 0;
    if (has_tokens && (!x || !log_a || !B || !C || !y)) return SSD_ERR_INVALID;
    const void* ptrs[] = {x, log_a, B, C, D, init_state, y, final_state, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    const size_t need = workspace_needed(d, chunk);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_ERR_INVALID;
    if (d->batch == 0) return SSD_OK;
    if (d->seqlen == 0 && !final_state) return SSD_OK;

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
    fl.Bm = B;
    fl.Cm = C;
    fl.D = D;
    fl.init = init_state;
    fl.y = y;
    fl.final_state = final_state;
    fl.scores = static_cast<float*>(workspace);
    fl.events = reinterpret_cast<hipEvent_t const*>(events);
    fl.n_events = events ? n_events : 0;
    fl.n_launches = n_launches;
    rc = ssd::launch_forward(fl, static_cast<hipStream_t>(stream));
    if (rc == -2) return SSD_ERR_UNSUPPORTED;
    return rc == 0 ? SSD_OK : SSD_ERR_HIP;
}

int ssd_step(const ssd_dims* d, float* state, const void* x_t, const float* log_a_t, const void* B_t,
             const void* C_t, const float* D, void* y_t, void* stream) {
    int rc = check_dims(d, false);
    if (rc != SSD_OK) return rc;
    if (d->headdim > 256 || 256 % d->headdim != 0) return SSD_ERR_UNSUPPORTED;
    if (d->batch == 0) return SSD_OK;
    if (!state || !x_t || !log_a_t || !B_t || !C_t || !y_t) return SSD_ERR_INVALID;
    const void* ptrs[] = {state, x_t, log_a_t, B_t, C_t, D, y_t};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    ssd::StepParams sp{state, x_t, log_a_t, B_t, C_t, D, y_t, d->nheads, d->ngroups,
                       (int)d->headdim, (int)d->dstate, d->decay == SSD_DECAY_DIAG ? 1 : 0};
    rc = ssd::launch_step(sp, d->dtype, d->batch * d->nheads, static_cast<hipStream_t>(stream));
    return rc == 0 ? SSD_OK : SSD_ERR_HIP;
}

const char* ssd_strerror(int code) {
    switch (code) {
        case SSD_OK: return "success";
        case SSD_ERR_INVALID: return "invalid argument (null pointer, bad dimension or workspace too small)";
        case SSD_ERR_UNSUPPORTED: return "unsupported configuration (chunk, dstate, headdim, dtype or decay kind)";
        case SSD_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case SSD_ERR_HIP: return "HIP runtime rejected a kernel launch";
        default: return "unknown error code";
    }
}

}  // extern "C"
