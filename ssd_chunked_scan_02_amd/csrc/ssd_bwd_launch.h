// Host-side launch interface of the backward pass (ssd_bwd.hip), between the C ABI (ssd_api.cpp)
// and its kernels.
#pragma once

#include "ssd_launch.h"

namespace ssd {

// The backward pass (ssd_bwd.hip), scalar or diagonal decay: inputs, the gradients it writes, and its
// workspace (the state entering every backward chunk, per-(batch, head) sums for dD, and for the
// diagonal decay the gradient of the state at every chunk's end, per-chunk decays, and the
// intra-chunk terms of dx, dB, dC and dlog a, per (b, t, h) row).
struct BwdParams {
    const void* x;
    const float* log_a;
    const void* Bm;
    const void* Cm;
    const float* D;
    const float* init;
    const void* dy;
    const float* dfinal;
    void* dx;
    float* dlog_a;
    float* dB;
    float* dC;
    float* dD;
    float* dinit;
    float* ckpt;
    float* dD_part;
    float* gst;    // diagonal decay: [B,H,nchunks,N,P] (the checkpoints' layout)
    float* elw;    // diagonal decay: [B,H,nchunks,N]
    float* dxi;    // diagonal decay: [B,T,H,P]
    float* dBi;    // diagonal decay: [B,T,H,N] (dCi, dcumi likewise)
    float* dCi;
    float* dcumi;
    int64_t batch, seqlen, nheads, ngroups;
    int nchunks;  // backward chunks (backward_chunk() tokens each)
    int64_t per_xcd, per_xcd_intra;
    // packed variable-length batch (null: batched layout), as in ForwardLaunch: the workspace keeps
    // the [batch][seqlen] layout, and each (sequence, head) covers its own chunks
    const int64_t* seq_off;
    int64_t total;
};
struct BackwardLaunch {
    int dtype;
    int decay;  // 0 scalar, 1 diagonal
    int64_t headdim, dstate;
    BwdParams p;
    // optional timing events, as in ForwardLaunch
    hipEvent_t const* events;
    int n_events;
    int* n_launches;
};
bool backward_shape_supported(int N, int P, int decay);
size_t backward_workspace_bytes(int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, int decay);
// Points p's workspace fields into ws (backward_workspace_bytes of it); p.batch, nheads and seqlen set.
void bind_backward_workspace(BwdParams& p, void* ws, int N, int P, int decay);
int backward_chunk();
// 0 on success, -1 when HIP rejects a launch, -2 for an unsupported shape.
int launch_backward(const BackwardLaunch& bl, hipStream_t stream);

// The discretised form's backward (ssd_backward_dt): its own arguments, and its workspace (log a,
// the scaled input, dx_in, dlog a, per-row sums (per row and state dim for dA_log with the
// diagonal decay), then the backward pass's own workspace).
struct DtBackwardArgs {
    const void* x;
    const float* dt;
    const float* dt_bias;
    const float* A_log;
    int scale_input;
    const float* D;
    const void* dy;
    void* dx;
    float* ddt;
    float* dA_log;
    float* ddt_bias;
    float* dD;
    void* workspace;
};
struct DtBackwardLayout {
    size_t la, xs, dxs, dla, ddt_rows, rowA, rowD, inner, total;
};
DtBackwardLayout dt_backward_layout(int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, int elem_bytes,
                                    bool scale_input, int decay);
int launch_backward_dt(const BackwardLaunch& bl, const DtBackwardArgs& a, hipStream_t stream);

}  // namespace ssd
