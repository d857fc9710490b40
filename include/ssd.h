/*
 * ssd.h - C ABI of libssd: the chunked Structured State-Space Duality (SSD) forward pass
 * and its single-token decode step, as HIP kernels for MI355X (gfx950).
 *
 * The operator (llms.blog "State Space Models and Mamba", sections "Continuous-to-Discrete
 * Discretization" and "The SSD Theoretical Equivalence"; per-state-dimension decay from
 * "On Structured State-Space Duality", ICML 2026 poster, abstract item (i)): for every batch
 * entry b and head h, with B/C group g = h / (H/G) ("Multi-Head State Space Layers"),
 *
 *     h_t = a_t * h_{t-1} + B_t x_t^T          a_t = exp(log_a[b,t,h])   (scalar decay)
 *                                              a_t = diag(exp(log_a[b,t,h,:]))  (diagonal)
 *     y_t = C_t^T h_t + D_h x_t
 *
 * with h an N x P fp32 state per (b, h), h_{-1} = init_state (or zeros).  ssd_forward
 * evaluates it chunk by chunk (aiwiki "State Space Duality", "Two algorithms for one
 * operator"; llms.blog "The Chunk-Wise SSD Algorithm"): inside a chunk of `chunk` tokens the
 * quadratic masked form (L o C B^T) X on matrix cores, between chunks one N x P state.
 *
 * Layouts: dense, row-major, last index fastest, no padding between rows.
 *     x, y          [B, T, H, P]    element type `dtype`
 *     log_a         [B, T, H] (SSD_DECAY_SCALAR) or [B, T, H, N] (SSD_DECAY_DIAG), fp32
 *     B, C          [B, T, G, N]    element type `dtype`
 *     D             [H] fp32, may be NULL (no skip term)
 *     init_state, final_state, state   [B, H, N, P] fp32
 *
 * Ownership: every pointer belongs to the caller; the library never allocates, frees or
 * retains device memory, and keeps no state between calls (one exception: the fixed scratch
 * array behind ssd_forward_noalloc, below).  Tensor pointers are DEVICE
 * pointers; `dims` is a HOST pointer read during the call only.  Work is enqueued on
 * `stream` (a hipStream_t passed as an opaque pointer; NULL = the default stream) and the
 * call returns without synchronising: outputs are valid once the stream has reached this
 * point.  Inputs must not alias outputs (except ssd_step's in-place state).
 *
 * Errors: every function returns 0 (SSD_OK) or a negative code, and every argument check
 * runs before any HIP call, so an invalid call has no effect.  Values are not checked:
 * log_a must be finite and <= 0 (a in (0, 1]); NaN/Inf inputs propagate to the outputs.
 * SSD_ERR_HIP reports a failed launch; faults during execution surface at the caller's
 * next synchronisation of the stream.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of x, B, C, y (log_a, D and states are always fp32). */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Shape of log_a: one decay per (b, t, h), or one per (b, t, h, n). */
typedef enum { SSD_DECAY_SCALAR = 0, SSD_DECAY_DIAG = 1 } ssd_decay;

typedef struct {
    int64_t batch;    /* B  >= 0 */
    int64_t seqlen;   /* T  >= 0 (ssd_step ignores it) */
    int64_t nheads;   /* H  >= 1 */
    int64_t ngroups;  /* G  >= 1, divides H */
    int64_t headdim;  /* P: 16, 32, 64 or 128 */
    int64_t dstate;   /* N: 16 (fp32 only), 32, 64, 128 or 256; N * P <= 16384 */
    int32_t dtype;    /* ssd_dtype */
    int32_t decay;    /* ssd_decay */
} ssd_dims;

enum {
    SSD_OK = 0,
    SSD_ERR_INVALID = -1,     /* NULL required pointer, bad dimension, workspace too small */
    SSD_ERR_UNSUPPORTED = -2, /* valid but not implemented: chunk, N, P or dtype combination */
    SSD_ERR_ALIGN = -3,       /* a tensor pointer is not 16-byte aligned */
    SSD_ERR_HIP = -4,         /* the HIP runtime rejected a launch */
    SSD_ERR_SCRATCH = -5      /* ssd_forward_noalloc: workspace larger than its fixed scratch */
};

/*
 * Bytes of device workspace ssd_forward needs for these dims and chunk length (0 when the
 * arguments are invalid or unsupported, or when no workspace is needed).  Pure host
 * arithmetic, no HIP call.
 */
size_t ssd_forward_workspace_bytes(const ssd_dims* dims, int chunk);

/*
 * Chunked SSD forward over a whole sequence (aiwiki "State Space Duality", "Two algorithms
 * for one operator"; llms.blog "The Chunk-Wise SSD Algorithm").
 *
 *   chunk         chunk length Q: 16, 32, 64, 128 or 256.  T need not be a multiple of Q:
 *                 the last chunk is then shorter (same operator, same result).
 *   D             [H] skip weights, or NULL for none.
 *   init_state    state entering token 0, or NULL for zeros.
 *   y             output [B,T,H,P] in `dtype` (fp32 accumulate, one rounding to bf16).
 *   final_state   state after token T-1, or NULL to skip writing it.
 *   workspace     device scratch of at least ssd_forward_workspace_bytes(dims, chunk) bytes
 *                 (may be NULL when that is 0); its contents are undefined afterwards.
 *   stream        hipStream_t as an opaque pointer (NULL = default stream).
 */
int ssd_forward(const ssd_dims* dims, const void* x, const float* log_a, const void* B,
                const void* C, const float* D, int chunk, const float* init_state, void* y,
                float* final_state, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssd_forward, and in addition has each of its kernel launches stamp caller-created
 * hipEvent_t handles (passed as opaque pointers), for timing each kernel live: launch k
 * records events[2k] when its dispatch starts and events[2k+1] when it ends (the stamps are
 * taken by the dispatch itself, so no extra packets sit between the kernels), and
 * hipEventElapsedTime(events[2k], events[2k+1]) is that kernel's run time.  Handles past
 * index 2L - 1 are left untouched; a NULL pair leaves that launch untimed.  *n_launches (a
 * HOST pointer, may be NULL) receives the number L of launches (L <= SSD_MAX_LAUNCHES).
 * With events non-NULL, n_events must be at least 2 * SSD_MAX_LAUNCHES, else the call fails
 * with SSD_ERR_INVALID before doing anything.  Launch order of the bf16 scalar-decay path:
 * prep (score tiles C B^T and operand layouts), then for a segmented walk the state-only
 * pass, then the chunk walk (states and outputs).  The diagonal-decay path's segmented walk runs
 * its state-only pass, the segment prefix and its walk.  The generic paths of ssd_forward_dt
 * (see below) run the discretisation first and, with a skip term and the input scale, a skip
 * pass last.
 */
#define SSD_MAX_LAUNCHES 4
int ssd_forward_profiled(const ssd_dims* dims, const void* x, const float* log_a, const void* B,
                         const void* C, const float* D, int chunk, const float* init_state,
                         void* y, float* final_state, void* workspace, size_t workspace_bytes,
                         void* stream, void* const* events, int n_events, int* n_launches);

/*
 * One decode step for every (b, h): the recurrence above for a single token, updating
 * `state` in place (llms.blog "The Duality of Inference and Training ...", item 1, linear
 * recurrence with O(1) memory per step).  dims->seqlen is ignored.
 *   state    [B,H,N,P] fp32, read and overwritten.
 *   x_t      [B,H,P];  log_a_t [B,H] or [B,H,N];  B_t, C_t [B,G,N];  D [H] or NULL;
 *   y_t      [B,H,P] output in `dtype`.
 */
int ssd_step(const ssd_dims* dims, float* state, const void* x_t, const float* log_a_t,
             const void* B_t, const void* C_t, const float* D, void* y_t, void* stream);

/*
 * The discretisation front-end, fused into the forward pass and the decode step (llms.blog
 * "State Space Models and Mamba": the zero-order-hold rule A-bar = exp(Delta A) of
 * "Continuous-to-Discrete Discretization"; the input-dependent step size, A-bar_t =
 * exp(Delta_t A) and B-bar_t = Delta_t B_t of "The Selection Mechanism").  In place of log_a
 * these entry points take the step-size pre-activation dt and compute, per (b, t, h):
 *
 *     Delta_t = softplus(dt[b,t,h] + dt_bias[h])        (dt_bias may be NULL: no bias)
 *     log a_t = -Delta_t * exp(A_log[h])                (SSD_DECAY_SCALAR; A_log [H])
 *     log a_t = -Delta_t * exp(A_log[h,n]) for each n   (SSD_DECAY_DIAG;   A_log [H, N])
 *
 * and, when scale_input is nonzero, the input term Delta_t B_t x_t^T in place of B_t x_t^T
 * (B-bar = Delta B).  The skip term D x_t always uses the raw x_t.  dt, dt_bias and A_log are
 * fp32 device tensors: dt [B,T,H] for the forward pass, [B,H] for the step.  Everything else
 * (layouts, ownership, streams, errors) is as for ssd_forward and ssd_step; the workspace size
 * differs, so it has its own query.  log a is never written to memory on the bf16 paths (scalar
 * decay with P = 64, N in {64, 128}, chunk in {64, 128, 256}; diagonal decay with N, P in
 * {32, 64}, chunk 64): their kernels form it from dt as they load each chunk.  Other shapes
 * first write log a (and Delta x, when scale_input) into the workspace, run the same walk, and
 * add the skip term afterwards.
 * Values: dt, dt_bias and A_log must be finite; Delta_t below the fp32 normal range (dt + bias
 * under about -87) is taken as 0 in the input term, and Delta_t above 2^64 is outside the range
 * the kernels' exact early exits assume.
 */
size_t ssd_forward_dt_workspace_bytes(const ssd_dims* dims, int chunk, int scale_input);

int ssd_forward_dt(const ssd_dims* dims, const void* x, const float* dt, const float* dt_bias,
                   const float* A_log, int scale_input, const void* B, const void* C,
                   const float* D, int chunk, const float* init_state, void* y,
                   float* final_state, void* workspace, size_t workspace_bytes, void* stream);

/* ssd_forward_dt with per-launch timing events, as ssd_forward_profiled. */
int ssd_forward_dt_profiled(const ssd_dims* dims, const void* x, const float* dt,
                            const float* dt_bias, const float* A_log, int scale_input,
                            const void* B, const void* C, const float* D, int chunk,
                            const float* init_state, void* y, float* final_state,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events, int n_events, int* n_launches);

/* ssd_step with the discretisation front-end: dt_t [B,H], A_log [H] or [H,N]. */
int ssd_step_dt(const ssd_dims* dims, float* state, const void* x_t, const float* dt_t,
                const float* dt_bias, const float* A_log, int scale_input, const void* B_t,
                const void* C_t, const float* D, void* y_t, void* stream);

/*
 * Packed variable-length batch.  dims->batch sequences lie one after another on one token axis
 * of total_tokens tokens: x [total,H,P], log_a [total,H] or [total,H,N], B, C [total,G,N] and
 * y [total,H,P], in the layouts and types of ssd_forward with the batch axis folded into the token
 * axis.  Sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1.  Each sequence runs the
 * recurrence by itself, from init_state[b] (zeros when init_state is NULL) to final_state[b]
 * (init_state, final_state [batch,H,N,P] fp32, optional): nothing passes from one sequence to the
 * next (llms.blog "State Space Models and Mamba", "Continuous-to-Discrete Discretization": the
 * recurrence starts from its initial state for each sequence).
 *   cu_seqlens: DEVICE memory, batch + 1 int64 values, 8-byte aligned, non-decreasing from 0 to
 *     total_tokens.  The kernels read it: a sequence's tokens are clamped into [0, total_tokens)
 *     and to its first dims->seqlen tokens, so malformed offsets give wrong outputs but never an
 *     access outside the tensors or the workspace.  The host does not read it.
 *   dims->seqlen: a bound on every sequence's length (the longest one's length is the natural
 *     choice).  Tokens past that bound, and tokens outside every sequence, are never written and
 *     enter no output.
 *   The bf16 scalar-decay fast path (head dim 64, N 64 or 128) has two forms.  Sequence by
 *     sequence: one walk per (sequence, head), as a batch; always taken when init_state or
 *     final_state is given.  As one sequence (init_state and final_state both NULL): the packed
 *     axis is walked like one long sequence of total_tokens tokens, segmented over the CUs, with
 *     the recurrence restarted at every sequence's first token (marked on the device from
 *     cu_seqlens, by the first kernel, or from 4096 sequences on by a launch of its own), so the
 *     work follows the token count, not the sequence count.
 *     The host takes the form with the shorter estimated walk from batch, total_tokens,
 *     dims->seqlen and the head count.  Either gives the same operator; outputs differ only in
 *     rounding.
 *   Workspace: the larger of the two forms' needs (a [batch][seqlen] batch's without the
 *     segmented walks, plus 4 bytes per sequence for up to 4096 sequences' order; and the batched
 *     layout of one sequence of batch * seqlen tokens with its segment states, plus 4 bytes per
 *     token of whole chunks).
 *   chunk, shapes, dtypes and decay kinds as ssd_forward.
 *   events, n_events, n_launches: as ssd_forward_profiled (NULL, 0, NULL: no timing).
 * Returns as ssd_forward; SSD_ERR_INVALID also for total_tokens < 0 or above batch * seqlen, or a
 * NULL or misaligned cu_seqlens with batch > 0.
 */
size_t ssd_forward_varlen_workspace_bytes(const ssd_dims* dims, int chunk);

int ssd_forward_varlen(const ssd_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                       const void* x, const float* log_a, const void* B, const void* C,
                       const float* D, int chunk, const float* init_state, void* y,
                       float* final_state, void* workspace, size_t workspace_bytes, void* stream,
                       void* const* events, int n_events, int* n_launches);

/* ssd_forward_varlen with the discretisation front-end, as ssd_forward_dt: dt [total,H], dt_bias
 * [H] (may be NULL), A_log [H] or [H,N], scale_input; the workspace from its own query. */
size_t ssd_forward_dt_varlen_workspace_bytes(const ssd_dims* dims, int chunk, int scale_input);

int ssd_forward_dt_varlen(const ssd_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                          const void* x, const float* dt, const float* dt_bias, const float* A_log,
                          int scale_input, const void* B, const void* C, const float* D, int chunk,
                          const float* init_state, void* y, float* final_state, void* workspace,
                          size_t workspace_bytes, void* stream, void* const* events, int n_events,
                          int* n_launches);

/*
 * The backward pass of ssd_forward: the gradients of L = <dy, y> + <dfinal,
 * final_state> with respect to every input, for training.  It is the chain rule through the
 * recurrence above, evaluated chunk by chunk (the state entering every chunk is recomputed into
 * the workspace, then a reverse walk carries dL/dh from chunk to chunk); the pages define the
 * operator, not its gradient.  The result is the gradient of the exact operator: it does not
 * depend on the forward pass's chunk length.
 *
 *   x, log_a, B, C, D, init_state   the forward pass's inputs (D and init_state may be NULL).
 *   dy            [B,T,H,P] in `dtype`: dL/dy.
 *   dfinal        [B,H,N,P] fp32 dL/dfinal_state, or NULL for zeros.
 *   dx            [B,T,H,P] output in `dtype`.
 *   dlog_a        [B,T,H] (or [B,T,H,N] for diagonal decay) fp32 output.
 *   dB, dC        [B,T,G,N] fp32 outputs (summed over the heads of each group).
 *   dD            [H] fp32 output, or NULL to skip it.
 *   dinit         [B,H,N,P] fp32 output dL/dinit_state, or NULL to skip it.
 *   workspace     device scratch of at least ssd_backward_workspace_bytes(dims) bytes: one fp32
 *                 N x P state per (batch, head, 32 tokens), plus 4 bytes per (batch, head).
 * Supported: SSD_DECAY_SCALAR with N in {16, 32, 64, 128}, or SSD_DECAY_DIAG with N in {16, 32,
 * 64} (dlog_a is then [B,T,H,N]); P in {16, 32, 64}; fp32 or bf16 (else SSD_ERR_UNSUPPORTED).  dB and dC are accumulated with atomic adds, so their last bits
 * may differ from run to run.
 */
size_t ssd_backward_workspace_bytes(const ssd_dims* dims);

int ssd_backward(const ssd_dims* dims, const void* x, const float* log_a, const void* B,
                 const void* C, const float* D, const float* init_state, const void* dy,
                 const float* dfinal, void* dx, float* dlog_a, float* dB, float* dC, float* dD,
                 float* dinit, void* workspace, size_t workspace_bytes, void* stream);

/* ssd_backward with per-launch timing events, as ssd_forward_profiled.  Launch order, scalar
 * decay: zeroing of dB and dC, the state checkpoints, the reverse walk, the dD reduction (when dD
 * is requested).  Diagonal decay: the per-chunk local kernel (which also clears dB and dC), the
 * scan over chunks, the state-terms kernel, the dD reduction (when dD is requested). */
int ssd_backward_profiled(const ssd_dims* dims, const void* x, const float* log_a, const void* B,
                          const void* C, const float* D, const float* init_state, const void* dy,
                          const float* dfinal, void* dx, float* dlog_a, float* dB, float* dC,
                          float* dD, float* dinit, void* workspace, size_t workspace_bytes,
                          void* stream, void* const* events, int n_events, int* n_launches);

/*
 * The backward pass of ssd_forward_varlen: a packed variable-length batch (the layouts, cu_seqlens,
 * total_tokens and dims->seqlen bound of ssd_forward_varlen), every sequence's gradients taken by
 * themselves: dx, dlog_a, dB, dC per packed token, dD summed over every sequence and head's tokens,
 * dinit [batch,H,N,P] per sequence (dfinal [batch,H,N,P] per sequence, may be NULL).  Shapes,
 * dtypes and decay kinds as ssd_backward; the workspace is ssd_backward's for these dims.
 * events, n_events, n_launches as ssd_backward_profiled (NULL, 0, NULL: no timing).  Offsets are
 * clamped as in ssd_forward_varlen.
 */
size_t ssd_backward_varlen_workspace_bytes(const ssd_dims* dims);

int ssd_backward_varlen(const ssd_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                        const void* x, const float* log_a, const void* B, const void* C,
                        const float* D, const float* init_state, const void* dy,
                        const float* dfinal, void* dx, float* dlog_a, float* dB, float* dC,
                        float* dD, float* dinit, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* events, int n_events, int* n_launches);

/*
 * The backward pass of ssd_forward_dt: the gradients of <dy, y> + <dfinal, final_state> with
 * respect to x, dt, A_log, dt_bias, B, C, D and init_state, by the chain rule through the
 * discretisation (Delta = softplus(dt + bias), log a = -Delta exp(A_log), and with scale_input the
 * input term Delta B x^T) around ssd_backward.
 *   A_log [H] (scalar decay) or [H,N] (dims->decay = SSD_DECAY_DIAG), as for ssd_forward_dt.
 *   ddt [B,T,H] fp32 (required); dA_log (A_log's shape) and ddt_bias [H] fp32 (NULL to skip each);
 *   dx, dB, dC, dD, dinit as for ssd_backward.
 *   workspace: at least ssd_backward_dt_workspace_bytes(dims, scale_input) bytes.
 * Supported shapes and dtypes as ssd_backward, for either decay kind.
 */
size_t ssd_backward_dt_workspace_bytes(const ssd_dims* dims, int scale_input);

int ssd_backward_dt(const ssd_dims* dims, const void* x, const float* dt, const float* dt_bias,
                    const float* A_log, int scale_input, const void* B, const void* C,
                    const float* D, const float* init_state, const void* dy, const float* dfinal,
                    void* dx, float* ddt, float* dA_log, float* ddt_bias, float* dB, float* dC,
                    float* dD, float* dinit, void* workspace, size_t workspace_bytes, void* stream);

/* ssd_backward_dt for a packed variable-length batch (the layouts, cu_seqlens, total_tokens and
 * dims->seqlen bound of ssd_forward_varlen; dt [total,H]): every sequence's gradients by themselves,
 * with ddt per packed token and dA_log, ddt_bias, dD summed over every sequence.  The workspace is
 * ssd_backward_dt's for these dims. */
size_t ssd_backward_dt_varlen_workspace_bytes(const ssd_dims* dims, int scale_input);

int ssd_backward_dt_varlen(const ssd_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                           const void* x, const float* dt, const float* dt_bias, const float* A_log,
                           int scale_input, const void* B, const void* C, const float* D,
                           const float* init_state, const void* dy, const float* dfinal, void* dx,
                           float* ddt, float* dA_log, float* ddt_bias, float* dB, float* dC, float* dD,
                           float* dinit, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssd_forward without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.  It runs
 * the same kernels as ssd_forward (same results, bit for bit) with the workspace placed in a
 * fixed array of ssd_noalloc_scratch_bytes() bytes (96 MiB) that the library holds on each GPU
 * it runs on, from the first use of the library's code on that GPU until the process ends.  The
 * call allocates and frees nothing.  Arguments are those of ssd_forward minus the workspace.
 *
 * Limit: a call whose ssd_forward_workspace_bytes(dims, chunk) exceeds the array fails with
 * SSD_ERR_SCRATCH before doing anything (the Mamba-2 layer shape, 8 x 2048 tokens x 24 heads at
 * N = 128, needs 12 MiB; one 65 536-token sequence of 32 heads, 58 MiB; 4 x 8192 tokens x 64 heads
 * in 8 groups, 176 MiB, which does not fit).
 * Races: every call on one GPU uses that GPU's one array, so calls that overlap in time on one
 * GPU (on different streams, or from several threads without ordering) corrupt each other's
 * workspace.  Calls ordered on one stream are safe: no call needs anything the previous one left
 * in the array.  The first call on each device looks up the array's device address (one HIP
 * runtime query, done before any launch); a failure there returns SSD_ERR_HIP.
 */
size_t ssd_noalloc_scratch_bytes(void);
int ssd_forward_noalloc(const ssd_dims* dims, const void* x, const float* log_a, const void* B,
                        const void* C, const float* D, int chunk, const float* init_state, void* y,
                        float* final_state, void* stream);

/* Static, human-readable description of a return code. */
const char* ssd_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
