// Host-side launch interface between the C ABI (ssd_api.cpp) and the kernels
// (ssd_kernels.hip).  Kernel parameter blocks are passed by value.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

struct ScoresParams {
    const void* Bm;
    const void* Cm;
    float* scores;
    int64_t seqlen;
    int64_t ngroups;
    int chunk;
    int nchunks;
    // packed variable-length batch (null: batched layout), as in ForwardLaunch
    const int64_t* seq_off;
    int64_t total;
};

struct WalkParams {
    const void* x;
    const float* log_a;
    const void* Bm;
    const void* Cm;
    const float* D;
    const float* scores;
    const float* init;
    void* y;
    float* final_state;
    int64_t batch, seqlen, nheads, ngroups;
    int chunk;
    int nchunks;
    int64_t per_xcd;
    // segmented walks (nseg > 1), as in Walk2Params
    int seg_chunks, nseg;
    float* seg_init;
    float* seg_state;
    float* seg_decay;
    // discretisation front-end (pipelined diagonal walk only; dt null otherwise): log a and
    // the input scale from dt, as in ForwardLaunch
    const float* dt;
    const float* dt_bias;
    const float* A_log;
    int scale_input;
    // packed variable-length batch (null: batched layout), as in ForwardLaunch
    const int64_t* seq_off;
    int64_t total;
};

struct StepParams {
    float* state;
    const void* x_t;
    const float* log_a_t;
    const void* B_t;
    const void* C_t;
    const float* D;
    void* y_t;
    int64_t nheads, ngroups;
    int headdim, dstate, diag;
    // discretisation front-end (dt_t non-null; log_a_t is then null), as in ForwardLaunch
    const float* dt_t;
    const float* dt_bias;
    const float* A_log;
    int scale_input;
};

struct PrepParams {
    const void* Bm;
    const void* Cm;
    const float* log_a;
    __bf16* pairs;  // score tile pairs, bf16, lane order
    __bf16* bt;     // B^T per chunk, tokens in MFMA K order
    __bf16* ct;     // C^T per chunk, MFMA lane order
    float* la_t;    // log a head-major: [batch][nheads][nchunks * chunk], 0 past the end
    // discretisation front-end (dt non-null; log_a is then null): log a from dt, and with
    // lg_t non-null log2 of the input scale softplus(dt + bias), laid out as la_t
    const float* dt;
    const float* dt_bias;
    const float* A_log;
    float* lg_t;
    int64_t seqlen;
    int64_t nheads;
    int64_t ngroups;
    int nchunks;
    int64_t nblk;  // batch * ngroups * nchunks
    int split;     // 1: two workgroups per block (see prep_kernel)
    // packed variable-length batch (null: batched layout), as in ForwardLaunch; with order non-null
    // the grid's first workgroups rank the sequences for the walk (order[rank] = b) and the blocks
    // follow them
    const int64_t* seq_off;
    int64_t total;
    int* order;
    // a packed batch walked as one sequence (flags non-null; the layout is then batch 1 with
    // seq_off null): the workgroups of group 0 that write the C^T and B^T fragments also write
    // their chunk's token flags (Walk2Params::tok_flags) from the batch's mark_nseq + 1 offsets
    // mark_off (at most kMarkLdsMax of them, staged in LDS after the B and C tiles), with
    // mark_bound the length bound and `total` the packed token count
    const int64_t* mark_off;
    int64_t mark_nseq;
    int64_t mark_bound;
    int* flags;
};

struct Walk2Params {
    const void* x;
    const float* la_t;  // log a head-major (PrepParams::la_t)
    const float* lg_t;  // log2 of the input scale head-major (PrepParams::lg_t), or null
    const __bf16* ct;   // C^T fragments (PrepParams::ct)
    const float* D;
    const __bf16* pairs;
    const __bf16* bt;
    const float* init;
    void* y;
    float* final_state;
    int64_t batch, seqlen, nheads, ngroups;
    int nchunks;
    int64_t per_xcd;
    // segmented walks (nseg > 1): chunks per segment, and per (segment, unit) the segment's local
    // final state from a zero start and its log2 decay
    int seg_chunks, nseg;
    float* seg_state;
    float* seg_decay;
    // packed variable-length batch (null: batched layout; never segmented), as in ForwardLaunch;
    // seq_order (or null): the sequences longest first, dealt round-robin to the XCDs by the walk
    const int64_t* seq_off;
    int64_t total;
    const int* seq_order;
    // a packed batch walked as one sequence (batch 1, seqlen = its token count): per token, bit 0
    // set where a sequence starts and bits 0 and 1 where a token lies outside every sequence (or
    // past the length bound); null otherwise
    const int* tok_flags;
};

// Everything one forward call needs, already validated.
struct ForwardLaunch {
    int dtype;  // 0 fp32, 1 bf16
    int decay;  // 0 scalar, 1 diagonal
    int64_t batch, seqlen, nheads, ngroups, headdim, dstate;
    int chunk, nchunks;
    const void* x;
    const float* log_a;
    // discretisation front-end (ssd_forward_dt): with dt non-null, log_a is null and the
    // kernels form log a = -softplus(dt + dt_bias) exp(A_log), and with scale_input the input
    // term's scale softplus(dt + dt_bias)
    const float* dt;
    const float* dt_bias;
    const float* A_log;
    int scale_input;
    const void* Bm;
    const void* Cm;
    const float* D;
    const float* init;
    void* y;
    float* final_state;
    float* scores;  // workspace
    // optional timing events (hipEvent_t): events[2k] and events[2k+1] take the start and end of
    // launch k
    hipEvent_t const* events;
    int n_events;
    int* n_launches;
    int first_launch;  // index of this call's first launch (a composed path continues the count)
    // Packed variable-length batch (ssd_forward_varlen): with seq_off non-null (device, batch + 1
    // offsets) sequence b is tokens seq_off[b] .. seq_off[b+1] of a packed token axis of `total`
    // tokens, seqlen bounds every length, and the workspace layouts are those of [batch][seqlen]
    // with no segmented walks.
    const int64_t* seq_off;
    int64_t total;
};

bool shape_supported(int dtype, int N, int P);
// Launch k of a forward call (k counts up).  With the caller's timing events the dispatch itself
// stamps events[2k] when it starts and events[2k+1] when it ends (hipExtLaunchKernel), so timing
// puts no extra packets between dependent kernels.  Updates *fl.n_launches; false on a HIP error.
// (L: ForwardLaunch or BackwardLaunch, anything with events, n_events and n_launches)
template <typename L, typename F, typename... Args>
bool launch_k(const L& fl, int& k, F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream, Args... args) {
    hipEvent_t start = nullptr, stop = nullptr;
    if (fl.events && 2 * k + 1 < fl.n_events) {
        start = fl.events[2 * k];
        stop = fl.events[2 * k + 1];
    }
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, start, stop, 0u, args...);
    ++k;
    if (fl.n_launches) *fl.n_launches = k;
    return hipGetLastError() == hipSuccess;
}
// The pipelined bf16 path (ssd_fast.hip) and its workspace.
bool fast_path_applies(int dtype, int decay, int N, int P, int chunk, int64_t nheads, int64_t ngroups);
// (with_lg: the workspace also holds log2 of the input scale, for ssd_forward_dt's scaled input)
size_t fast_workspace_bytes(int64_t batch, int64_t nheads, int64_t ngroups, int64_t seqlen, int N, int chunk,
                            bool with_lg = false, bool varlen = false);
int launch_forward_fast(const ForwardLaunch& fl, hipStream_t stream);
// The diagonal-decay walk (ssd_diag.hip): LDS bytes (0 = unsupported) and launch.
size_t diag_lds_bytes(int dtype, int N, int P, int chunk);
int launch_forward_diag(const ForwardLaunch& fl, hipStream_t stream);
// (varlen: a packed variable-length batch, never segmented)
size_t diag_workspace_bytes(int dtype, int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, int chunk,
                            bool varlen = false);
bool diag_pipe_applies(int dtype, int N, int P, int chunk);
// Segment prefix of a segmented walk (ssd_fast.hip): per_n = 1 for one decay per state row.
int launch_seg_prefix(const ForwardLaunch& fl, int& k, const float* init, float* seg_init, const float* seg_state,
                      const float* seg_decay, int64_t units, int N, int P, int nseg, int per_n, hipStream_t stream);
size_t walk_lds_bytes(int dtype, int N, int P, int chunk);
size_t scores_bytes(int64_t batch, int64_t ngroups, int64_t nchunks, int chunk);
// 0 on success, -1 when HIP rejects a launch, -2 for an unsupported shape.
int launch_forward(const ForwardLaunch& fl, hipStream_t stream);
int launch_step(const StepParams& sp, int dtype, int64_t units, hipStream_t stream);

// ssd_forward_dt on the paths whose kernels form log a from dt themselves (the bf16 scalar fast
// path and the pipelined diagonal walk).  Other shapes take the generic composition below.
inline bool discretization_fused(int dtype, int decay, int N, int P, int chunk, int64_t nheads, int64_t ngroups) {
    return decay == 1 ? diag_pipe_applies(dtype, N, P, chunk)
                      : fast_path_applies(dtype, decay, N, P, chunk, nheads, ngroups);
}
// Workspace of the generic composition: the walk's own workspace, then log a [B,T,H(,N)] fp32,
// then (scale_input) the scaled input softplus(dt + bias) x [B,T,H,P] in the element type, each
// part starting on a 256-byte boundary.
struct DtGenericLayout {
    size_t la, xs, total;
};
inline DtGenericLayout dt_generic_layout(size_t own, int64_t batch, int64_t seqlen, int64_t nheads, int64_t per_head,
                                         int64_t headdim, int elem_bytes, bool scale_input) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t tokens = (size_t)batch * (size_t)seqlen * (size_t)nheads;
    DtGenericLayout l;
    l.la = up(own);
    l.xs = up(l.la + tokens * (size_t)per_head * 4);
    l.total = scale_input ? l.xs + tokens * (size_t)headdim * (size_t)elem_bytes : l.xs;
    return l;
}
// Bytes of the walk's own workspace on the generic (unfused) path of these dims.
size_t generic_workspace_bytes(int dtype, int decay, int64_t batch, int64_t nheads, int64_t ngroups,
                               int64_t seqlen, int N, int P, int chunk);

constexpr size_t kMaxLds = 160 * 1024;

// The fixed per-device scratch array of ssd_forward_noalloc (ssd_noalloc.hip): its size, and the
// device address of the current device's copy (null with *hip_rc set on failure).
size_t noalloc_scratch_bytes();
void* noalloc_scratch(int* hip_rc);

// Segmented walks: with few (batch, head) units on a long sequence (at most half as many as the
// 256 CUs), each sequence is split into segments of at least 4 chunks so that about `target`
// workgroups walk (one per CU per round).  Returns the number of segments and sets *seg_chunks
// (chunks per segment; the last segment may be shorter).
inline int walk_segments(int64_t units, int64_t nchunks, int64_t target, int* seg_chunks) {
    constexpr int64_t kMinChunks = 4, kCUs = 256;
    int64_t nseg = 1;
    if (units > 0 && units * 2 <= kCUs && nchunks >= 2 * kMinChunks)
        nseg = (target / units < nchunks / kMinChunks) ? target / units : nchunks / kMinChunks;
    const int64_t per = (nchunks + nseg - 1) / nseg;
    *seg_chunks = (int)(per > 0 ? per : 1);
    return (int)(per > 0 ? (nchunks + per - 1) / per : 1);
}

}  // namespace ssd
