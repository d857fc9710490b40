// HIP kernels of the SSD backward pass (scalar decay), for gfx950 (MI355X).
//
// The gradient of L = <dy, y> + <dfinal, final> through the chunked forward pass, with the
// state carried between chunks.  Inside a chunk of Q tokens, with cum the running sum of log a
// (inclusive, restarting at the chunk), L_ts = exp(cum_t - cum_s) for s <= t (0 above),
// S = C B^T, e_t = exp(cum_t), w_s = exp(cum_last - cum_s), H the state entering the chunk and
// G the gradient of the state leaving it (dL/dh at the chunk's last token, from everything
// after it):
//   y_t  = sum_{s <= t} S_ts L_ts x_s + e_t C_t H + D x_t,     H_out = e_last H + sum_s w_s B_s x_s^T
// so that, with DYX_ts = dy_t . x_s and M_ts = S_ts L_ts DYX_ts,
//   dx_s   = sum_t (S o L)_ts dy_t + w_s B_s^T G + D dy_s
//   dB_s  += sum_t (L o DYX)_ts C_t + w_s G x_s                 (summed over the group's heads)
//   dC_t  += sum_s (L o DYX)_ts B_s + e_t H dy_t
//   dcum_t = sum_s M_ts - sum_t' M_t't + e_t C_t . (H dy_t) - w_t B_t . (G x_t)
//            + [t = last] (e_last <G, H> + sum_s w_s B_s . (G x_s))
//   dlog a_j = sum_{t >= j in the chunk} dcum_t
//   G_in   = e_last G + sum_t e_t C_t dy_t^T                    (the gradient entering the chunk)
// These are the chain rule through the chunk-wise form of aiwiki "State Space Duality" ("Two
// algorithms for one operator") and llms.blog "The Chunk-Wise SSD Algorithm"; the pages print no
// backward pass.
//
//   bwd_states_kernel  one workgroup per (batch, head) walks forward and writes the state entering
//                      every chunk (the checkpoints), the state kept in MFMA accumulators.
//   bwd_walk_kernel    one workgroup per (batch, head) walks the chunks last to first with G in
//                      accumulators, forms the chunk's gradients from fp32 MFMA products of LDS
//                      tiles, and adds dB and dC into the group's rows with atomic adds.
//   bwd_reduce_kernel  dD over the batch from the walk's per-(batch, head) partial sums.
// The backward chunk (32 tokens) is independent of the forward pass's: the gradient of the
// operator does not depend on how it is chunked.
#include <algorithm>
#include <type_traits>

#include "ssd_common.h"
#include "ssd_bwd_launch.h"

namespace ssd {
namespace {

constexpr int kBQ = 32;       // tokens per backward chunk
constexpr int kBwdCUs = 256;  // compute units: the persistent kernels' workgroup count

// acc += A B for one 16x16 tile (fp32 MFMA 16x16x4; lane l gives A(l % 16, k + l / 16) and
// B(k + l / 16, l % 16) and holds rows 4 (l / 16) + i, column l % 16 of the tile).  Element
// (m, k) of A is a[m * am + k * ak]; element (k, n) of B is b[k * bk + n * bn].
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const float* a, int am, int ak, const float* b, int bk, int bn,
                                          int K, int lane) {
    const int r = lane % 16, g = lane / 16;
#pragma unroll 4
    for (int k = 0; k < K; k += 4) acc = mfma_f32(a[r * am + (k + g) * ak], b[(k + g) * bk + r * bn], acc);
    return acc;
}

__device__ __forceinline__ double softplus_ct(double v) { return softplus(v); }
__device__ __forceinline__ float softplus_ct(float v) { return softplusf(v); }

// Sum over the 16 lanes of a lane group (the 16 columns of one accumulator row).
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off, 16);
    return v;
}

// element j of a 16-byte piece as fp32
template <typename T> __device__ __forceinline__ float piece_elem(uint4 u, int j);
template <> __device__ __forceinline__ float piece_elem<__bf16>(uint4 u, int j) { return (float)as_bf16x8(u)[j]; }
template <> __device__ __forceinline__ float piece_elem<float>(uint4 u, int j) { return as_f32x4(u)[j]; }

constexpr int kBWaves = 8;                     // waves per backward workgroup
constexpr int kBThreads = kBWaves * kWave;

template <int N, int P>
struct BwdShape {
    static constexpr int Q = kBQ, QS = Q + 1, NS = N + 1, PS = P + 1;
    static constexpr int NB = N / 16, PB = P / 16, QB = Q / 16;
    static constexpr int NTILE = NB * PB, TPW = (NTILE + kBWaves - 1) / kBWaves;  // state tiles per wave
    // walk LDS (floats): X, dY [Q][PS]; B, C [Q][NS]; S o L, L o DYX, DYX [Q][QS]; H, G [N][PS];
    // e, w, row sums and column sums of M [Q]; row partial sums of B . (G x) and C . (H dy)
    // [Q][NB] each; reduction [kBWaves]  (the running sums in a static array of their own type)
    static constexpr size_t walk_floats = (size_t)2 * Q * PS + 2 * Q * NS + 3 * Q * QS + 2 * N * PS + 4 * Q +
                                          2 * Q * NB + kBWaves;
    static constexpr size_t walk_lds = walk_floats * 4;
    // states LDS (floats): w o B [Q][NS], X [Q][PS]
    static constexpr size_t states_lds = ((size_t)Q * NS + Q * PS) * 4;
};

// One chunk's rows of a [.., rows, width] tensor in 16-byte pieces, a chunk ahead of their use:
// piece u of the chunk is row u / (width / VE), elements VE (u % (width / VE)) .. + VE; rows at
// or past len are zeros.  Each of the NT threads holds pieces tid + NT i.
template <typename T, int ROWS, int WIDTH, int NT = kBThreads>
struct ChunkRows {
    static constexpr int VE = 16 / (int)sizeof(T), PER_ROW = WIDTH / VE, PIECES = ROWS * PER_ROW;
    static constexpr int PT = (PIECES + NT - 1) / NT;
    uint4 v[PT];
    // row r of the chunk starts at base + r * stride (elements)
    __device__ void load(const T* base, int64_t stride, int len, int tid) {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + NT * i, r = u / PER_ROW, c = (u % PER_ROW) * VE;
            v[i] = (u < PIECES && r < len) ? ld16(base + r * stride + c) : uint4{0u, 0u, 0u, 0u};
        }
    }
    // into an fp32 LDS tile with row stride ld
    __device__ void stage(float* dst, int ld, int tid) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + NT * i, r = u / PER_ROW, c = (u % PER_ROW) * VE;
            if (u < PIECES)
#pragma unroll
                for (int j = 0; j < VE; ++j) dst[r * ld + c + j] = piece_elem<T>(v[i], j);
        }
    }
    __device__ float elem(int i, int j) const { return piece_elem<T>(v[i], j); }
    // as they are, into a tile of the input type with row stride ld (16-byte aligned rows)
    __device__ void stage_raw(T* dst, int ld, int tid) const {
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + NT * i, r = u / PER_ROW, c = (u % PER_ROW) * VE;
            if (u < PIECES) st16(dst + r * ld + c, v[i]);
        }
    }
};

// Running sum of log a over one chunk from la_v (token tid's log a in lanes tid < Q of wave 0, 0
// past the chunk's end), into cum[0..Q); then e = exp(cum) and w = exp(cum_last - cum).  CT is
// double for fp32 inputs (as the forward's generic path), and cum keeps it.
template <typename CT>
__device__ __forceinline__ void chunk_factors(float la_v, CT* cum, float* e, float* w, int tid) {
    if (tid < kWave) {
        CT v = tid < kBQ ? (CT)la_v : (CT)0;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const CT o = __shfl_up(v, off, kWave);
            if (tid >= off) v += o;
        }
        const CT last = __shfl(v, kBQ - 1, kWave);
        if (tid < kBQ) {
            cum[tid] = v;
            e[tid] = (float)exp(v);
            w[tid] = (float)exp(last - v);
        }
    }
}

// ---------------------------------------------------------------------------------------
template <typename T, int N, int P>
__global__ void __launch_bounds__(kBThreads) bwd_states_kernel(BwdParams prm) {
    using S = BwdShape<N, P>;
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    constexpr int Q = S::Q, NS = S::NS, PS = S::PS, PB = S::PB, NTILE = S::NTILE, TPW = S::TPW;
    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen, units = prm.batch * H;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, units);
    if (unit < 0) return;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
    // (the sequence's own chunks; the checkpoints keep the stride of prm.nchunks)
    const int nch = prm.seq_off ? (int)((sq.len + kBQ - 1) / kBQ) : prm.nchunks;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, lg = lane / 16, l16 = lane % 16;
    extern __shared__ __align__(16) unsigned char smem[];
    float* Bw = reinterpret_cast<float*>(smem);  // w o B [Q][NS]
    float* Xs = Bw + Q * NS;                     // [Q][PS]
    __shared__ CT cum[kBQ];
    __shared__ float e_unused[kBQ], w_s[kBQ];
    const T* xg = static_cast<const T*>(prm.x);
    const T* Bg = static_cast<const T*>(prm.Bm);

    f32x4 hs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        hs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wave + kBWaves * j;
        if (tile < NTILE && prm.init) {
            const int nb = tile / PB, pb = tile % PB;
#pragma unroll
            for (int i = 0; i < 4; ++i) hs[j][i] = prm.init[(unit * N + 16 * nb + 4 * lg + i) * P + 16 * pb + l16];
        }
    }
    ChunkRows<T, Q, N> rb;
    ChunkRows<T, Q, P> rx;
    float rla = 0.f;
    auto load = [&](int c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        rb.load(Bg + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rx.load(xg + ((sq.row0 + t0) * H + h) * P, H * P, len, tid);
        rla = tid < len && tid < Q ? prm.log_a[(sq.row0 + t0 + tid) * H + h] : 0.f;
    };
    if (nch > 0) load(0);
    for (int c = 0; c < nch; ++c) {
        // the checkpoint: the state entering chunk c
        float* ck = prm.ckpt + (unit * prm.nchunks + c) * (int64_t)N * P;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
#pragma unroll
                for (int i = 0; i < 4; ++i) ck[(16 * nb + 4 * lg + i) * P + 16 * pb + l16] = hs[j][i];
            }
        }
        chunk_factors<CT>(rla, cum, e_unused, w_s, tid);
        lds_barrier();
        rb.stage(Bw, NS, tid);
        rx.stage(Xs, PS, tid);
        lds_barrier();
        // w o B in place (rows past the end are zero already)
        for (int i = tid; i < Q * N; i += kBThreads) Bw[(i / N) * NS + i % N] *= w_s[i / N];
        const float el = (float)exp(cum[Q - 1]);
        lds_barrier();
        if (c + 1 < nch) load(c + 1);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                hs[j] = tile_mma(hs[j] * el, Bw + 16 * nb, 1, NS, Xs + 16 * pb, PS, 1, Q, lane);
            }
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------------------
template <typename T, int N, int P>
__global__ void __launch_bounds__(kBThreads) bwd_walk_kernel(BwdParams prm) {
    using S = BwdShape<N, P>;
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    constexpr int Q = S::Q, QS = S::QS, NS = S::NS, PS = S::PS, NB = S::NB, PB = S::PB, QB = S::QB;
    constexpr int NTILE = S::NTILE, TPW = S::TPW;
    static_assert(2 * QB * QB <= kBWaves, "one S o L or DYX tile per wave");
    static_assert(Q * 16 == kBThreads, "row and column sums: 16 threads per row");
    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen, units = prm.batch * H;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, units);
    if (unit < 0) return;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
    // (the sequence's own chunks; the checkpoints keep the stride of prm.nchunks)
    const int nch = prm.seq_off ? (int)((sq.len + kBQ - 1) / kBQ) : prm.nchunks;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, lg = lane / 16, l16 = lane % 16;

    extern __shared__ __align__(16) unsigned char smem[];
    float* Xs = reinterpret_cast<float*>(smem);  // [Q][PS]
    float* Ys = Xs + Q * PS;                     // dy [Q][PS]
    float* Bs = Ys + Q * PS;                     // [Q][NS]
    float* Cs = Bs + Q * NS;                     // [Q][NS]
    float* Am = Cs + Q * NS;                     // S o L [Q][QS] (rows t, columns s)
    float* Wm = Am + Q * QS;                     // L o DYX [Q][QS]
    float* Dm = Wm + Q * QS;                     // DYX [Q][QS]
    float* Hs = Dm + Q * QS;                     // H [N][PS]
    float* Gs = Hs + N * PS;                     // G [N][PS]
    float* ev = Gs + N * PS;
    float* wv = ev + Q;
    float* rowM = wv + Q;           // sum_s M_ts
    float* colM = rowM + Q;         // sum_t M_ts
    float* partB = colM + Q;        // [Q][NB]: B_s . (G x_s) over 16-column pieces
    float* partC = partB + Q * NB;  // [Q][NB]: C_t . (H dy_t)
    float* red = partC + Q * NB;    // [kBWaves]
    __shared__ CT cum[kBQ];

    const T* xg = static_cast<const T*>(prm.x);
    const T* yg = static_cast<const T*>(prm.dy);
    const T* Bg = static_cast<const T*>(prm.Bm);
    const T* Cg = static_cast<const T*>(prm.Cm);
    T* dxg = static_cast<T*>(prm.dx);
    const float dskip = prm.D ? prm.D[h] : 0.f;

    // G, the gradient of the state leaving the current chunk, in accumulators (tiles of the
    // N x P state dealt to the waves) and in Gs
    f32x4 gs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        gs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wave + kBWaves * j;
        if (tile < NTILE && prm.dfinal) {
            const int nb = tile / PB, pb = tile % PB;
#pragma unroll
            for (int i = 0; i < 4; ++i) gs[j][i] = prm.dfinal[(unit * N + 16 * nb + 4 * lg + i) * P + 16 * pb + l16];
        }
    }
    auto write_g = [&]() {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
#pragma unroll
                for (int i = 0; i < 4; ++i) Gs[(16 * nb + 4 * lg + i) * PS + 16 * pb + l16] = gs[j][i];
            }
        }
    };
    write_g();
    float dD_acc = 0.f;

    // the next chunk's inputs, a chunk ahead (chunks run last to first)
    ChunkRows<T, Q, P> rx, ry;
    ChunkRows<T, Q, N> rb, rc;
    ChunkRows<float, N, P> rh;
    float rla = 0.f;
    auto load = [&](int c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        rx.load(xg + ((sq.row0 + t0) * H + h) * P, H * P, len, tid);
        ry.load(yg + ((sq.row0 + t0) * H + h) * P, H * P, len, tid);
        rb.load(Bg + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rc.load(Cg + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rh.load(prm.ckpt + (unit * prm.nchunks + c) * (int64_t)N * P, P, N, tid);
        rla = tid < len && tid < Q ? prm.log_a[(sq.row0 + t0 + tid) * H + h] : 0.f;
    };
    if (nch > 0) load(nch - 1);

    for (int c = nch - 1; c >= 0; --c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        // ---- 1. the chunk's x, dy, B, C and entering state into LDS (zeros past the end)
        rx.stage(Xs, PS, tid);
        ry.stage(Ys, PS, tid);
        rb.stage(Bs, NS, tid);
        rc.stage(Cs, NS, tid);
        rh.stage(Hs, PS, tid);
#pragma unroll
        for (int i = 0; i < ChunkRows<T, Q, P>::PT; ++i)
#pragma unroll
            for (int j = 0; j < ChunkRows<T, Q, P>::VE; ++j) dD_acc += rx.elem(i, j) * ry.elem(i, j);
        chunk_factors<CT>(rla, cum, ev, wv, tid);
        lds_barrier();
        if (c > 0) load(c - 1);

        // ---- 2. S o L (waves 0 .. 3) and DYX, L o DYX (waves 4 .. 7), one 16 x 16 tile (tb, sb) each:
        //         rows t, columns s
        {
            const int job = wave % (QB * QB), tb = job / QB, sb = job % QB;
            const bool scores = wave < QB * QB;
            const f32x4 v = scores ? tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Cs + 16 * tb * NS, NS, 1, Bs + 16 * sb * NS, 1,
                                              NS, N, lane)
                                   : tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Ys + 16 * tb * PS, PS, 1, Xs + 16 * sb * PS, 1,
                                              PS, P, lane);
            const int s = 16 * sb + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * lg + i;
                const float L = s <= t ? (float)exp(cum[t] - cum[s]) : 0.f;
                if (scores) {
                    Am[t * QS + s] = v[i] * L;
                } else {
                    Wm[t * QS + s] = v[i] * L;
                    Dm[t * QS + s] = v[i];
                }
            }
        }
        lds_barrier();

        // ---- 3. row and column sums of M = (S o L) o DYX (16 threads per row or column); dx,
        //         dB, dC and the state terms of dcum, tiles dealt to the waves
        {
            const int r = tid / 16, j = tid % 16;
            float rs = 0.f, cs = 0.f;
#pragma unroll
            for (int k = 2 * j; k < 2 * j + 2; ++k) {
                rs += Am[r * QS + k] * Dm[r * QS + k];
                cs += Am[k * QS + r] * Dm[k * QS + r];
            }
            rs = group16_sum(rs);
            cs = group16_sum(cs);
            if (j == 0) {
                rowM[r] = rs;
                colM[r] = cs;
            }
        }
        for (int tile = wave; tile < QB * PB; tile += kBWaves) {
            const int sb = tile / PB, pb = tile % PB;
            // sum_t (S o L)_ts dy_t: A(s, t) = Am[t][s]
            const f32x4 acc = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Am + 16 * sb, 1, QS, Ys + 16 * pb, PS, 1, Q, lane);
            // B_s^T G: A(s, n) = Bs[s][n], B(n, p) = Gs[n][p]
            const f32x4 bg = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Bs + 16 * sb * NS, NS, 1, Gs + 16 * pb, PS, 1, N, lane);
            const int p = 16 * pb + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * sb + 4 * lg + i;
                const float v = acc[i] + wv[s] * bg[i] + dskip * Ys[s * PS + p];
                if (s < len) dxg[((sq.row0 + t0 + s) * H + h) * P + p] = from_f32<T>(v);
            }
        }
        for (int tile = wave; tile < QB * NB; tile += kBWaves) {
            const int sb = tile / NB, nb = tile % NB;
            // dB: sum_t (L o DYX)_ts C_t (A(s, t) = Wm[t][s], B(t, n) = Cs[t][n]) + w_s G x_s
            const f32x4 acc = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Wm + 16 * sb, 1, QS, Cs + 16 * nb, NS, 1, Q, lane);
            const f32x4 gx = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Xs + 16 * sb * PS, PS, 1, Gs + 16 * nb * PS, 1, PS, P,
                                      lane);
            // dC: sum_s (L o DYX)_ts B_s (A(t, s) = Wm[t][s], B(s, n) = Bs[s][n]) + e_t H dy_t
            const f32x4 acc2 = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Wm + 16 * sb * QS, QS, 1, Bs + 16 * nb, NS, 1, Q,
                                        lane);
            const f32x4 hd = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Ys + 16 * sb * PS, PS, 1, Hs + 16 * nb * PS, 1, PS, P,
                                      lane);
            const int n = 16 * nb + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * sb + 4 * lg + i;  // (the row: s for dB, t for dC)
                if (s < len) {
                    atomicAdd(prm.dB + ((sq.row0 + t0 + s) * G + g) * N + n, acc[i] + wv[s] * gx[i]);
                    atomicAdd(prm.dC + ((sq.row0 + t0 + s) * G + g) * N + n, acc2[i] + ev[s] * hd[i]);
                }
                const float pbv = group16_sum(Bs[s * NS + n] * gx[i]);
                const float pcv = group16_sum(Cs[s * NS + n] * hd[i]);
                if (l16 == 0) {
                    partB[s * NB + nb] = pbv;
                    partC[s * NB + nb] = pcv;
                }
            }
        }
        // <G, H>, block-wide
        float gh = 0.f;
        for (int i = tid; i < N * P; i += kBThreads) gh += Gs[(i / P) * PS + i % P] * Hs[(i / P) * PS + i % P];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) gh += __shfl_xor(gh, off, kWave);
        if (lane == 0) red[wave] = gh;
        lds_barrier();

        // ---- 4. dcum and dlog a as its reverse running sum (wave 0); the gradient entering the
        //         chunk, G <- e_last G + sum_t e_t C_t dy_t^T (every wave)
        const float el = ev[Q - 1];
        if (tid < kWave) {
            float d = 0.f, wpb = 0.f;
            if (tid < Q) {
                const int t = tid;
                float pb_ = 0.f, pc_ = 0.f;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    pb_ += partB[t * NB + nb];
                    pc_ += partC[t * NB + nb];
                }
                d = rowM[t] - colM[t] + ev[t] * pc_ - wv[t] * pb_;
                wpb = wv[t] * pb_;
            }
            // the last token's term: e_last <G, H> + sum_s w_s B_s . (G x_s)
            float ws = wpb;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off, kWave);
            if (tid == Q - 1) {
                float ghs = 0.f;
#pragma unroll
                for (int k = 0; k < kBWaves; ++k) ghs += red[k];
                d += el * ghs + ws;
            }
            // reverse inclusive running sum over t
            float r = tid < Q ? d : 0.f;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float o = __shfl_down(r, off, kWave);
                if (tid + off < kWave) r += o;
            }
            if (tid < len) prm.dlog_a[(sq.row0 + t0 + tid) * H + h] = r;
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                // A(n, t) = e_t Cs[t][n], B(t, p) = Ys[t][p]
                f32x4 acc = gs[j] * el;
                const int r = lane % 16, gq = lane / 16;
#pragma unroll 4
                for (int k = 0; k < Q; k += 4)
                    acc = mfma_f32(Cs[(k + gq) * NS + 16 * nb + r] * ev[k + gq], Ys[(k + gq) * PS + 16 * pb + r], acc);
                gs[j] = acc;
            }
        }
        lds_barrier();  // every read of Gs, Hs and the chunk tiles above is done
        write_g();
    }
    lds_barrier();
    if (prm.dinit) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
#pragma unroll
                for (int i = 0; i < 4; ++i) prm.dinit[(unit * N + 16 * nb + 4 * lg + i) * P + 16 * pb + l16] = gs[j][i];
            }
        }
    }
    // dy . x over the unit, for dD
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dD_acc += __shfl_xor(dD_acc, off, kWave);
    if (lane == 0) red[wave] = dD_acc;
    lds_barrier();
    if (tid == 0) {
        float s = 0.f;
        for (int k = 0; k < kBWaves; ++k) s += red[k];
        prm.dD_part[unit] = s;
    }
}

// ---------------------------------------------------------------------------------------
// bf16 inputs (N in {32, 64, 128}, P in {32, 64}): the same two passes with every tile product a
// bf16 MFMA (16x16x32) on bf16 LDS tiles.  Operands that contract along a tile's rows come from the
// transposing LDS read, the others from one 16-byte read per lane.  The products whose results go to
// memory (the state, dx, dB, dC, G) are formed transposed, so that each accumulator lane holds four
// consecutive elements of a row in memory.  The checkpoints are stored in bf16: H only enters bf16
// products and <G, H>.  The state and its gradient stay fp32 in the accumulators, and the row and
// column sums of M that dlog a needs come from fp32 copies of the S o L and DYX tiles.  Rounded to
// bf16 for the products: S o L, L o DYX, H, G, w o B and e o C (x, dy, B and C are bf16 already).
// The forward pass rounds S o L and H the same way.
template <int N, int P>
struct BwdBf16Shape {
    static constexpr int Q = kBQ, NB = N / 16, PB = P / 16, QB = Q / 16, QF = Q + 1;
    static constexpr int XS = P + 16, NSB = N + 8, QSB = Q + 16;  // bf16 row strides (elements)
    static constexpr int NTILE = NB * PB, TPW = (NTILE + kBWaves - 1) / kBWaves;
    // checkpoint pass: w o B [Q][NSB], x [Q][XS]
    static constexpr size_t states_lds = ((size_t)Q * NSB + (size_t)Q * XS) * 2;
    // walk: x, dy [Q][XS]; B, C [Q][NSB]; S o L, L o DYX [Q][QSB]; H, G [N][XS] (bf16); then S o L,
    // DYX [Q][QF], e, w, row and column sums of M [Q], the partial row sums of B . (G x) and
    // C . (H dy) [Q][NB] each, and the reduction [kBWaves] (fp32)
    static constexpr size_t bf_elems = (size_t)2 * Q * XS + 2 * Q * NSB + 2 * Q * QSB + 2 * N * XS;
    static constexpr size_t f_floats = (size_t)2 * Q * QF + 4 * Q + 2 * Q * NB + kBWaves;
    static constexpr size_t walk_lds = bf_elems * 2 + f_floats * 4;
    static_assert(bf_elems % 8 == 0, "fp32 part 16-byte aligned");
};

template <int N, int P>
constexpr bool bwd_bf16_shape() {
    return (N == 32 || N == 64 || N == 128) && (P == 32 || P == 64);
}

// Lane-to-lane moves inside 16-lane rows with DPP (no LDS round trip): the source lane's value
// under pattern CTRL for the rows in ROWS, 0 where the pattern has no source lane.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float bdpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
// Sum over the 16 lanes of a row, in every lane: swap neighbours, swap pairs, mirror each half,
// mirror the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += bdpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += bdpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += bdpp<0x141>(v);  // row_half_mirror
    v += bdpp<0x140>(v);  // row_mirror
    return v;
}
// Sum over the wave (the same value in every lane): row sums, then the four rows' from lanes 0, 16,
// 32 and 48.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = row16_sum(v);
    auto at = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
    return (at(0) + at(16)) + (at(32) + at(48));
}
// chunk_factors for fp32 running sums, with the scan over the chunk's 32 tokens in DPP steps (row
// shifts, then row 0's total into row 1) and the hardware exponential.
__device__ __forceinline__ void chunk_factors_dpp(float la_v, float* cum, float* e, float* w, int tid) {
    static_assert(kBQ == 32, "two 16-lane rows");
    if (tid < kWave) {
        float v = tid < kBQ ? la_v : 0.f;
        v += bdpp<0x111>(v);       // row_shr:1
        v += bdpp<0x112>(v);       // row_shr:2
        v += bdpp<0x114>(v);       // row_shr:4
        v += bdpp<0x118>(v);       // row_shr:8
        v += bdpp<0x142, 0xa>(v);  // row_bcast:15 into row 1
        const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kBQ - 1));
        if (tid < kBQ) {
            cum[tid] = v;
            e[tid] = __expf(v);
            w[tid] = __expf(last - v);
        }
    }
}

// An MFMA operand contracting over rows k0 .. k0 + 31 of a row-major bf16 LDS tile [k][col]: lane
// (g, i) receives tile[k0 + 8 g + j][col0 + i], j = 0..7 (two transposing reads, ds_read_b64_tr_b16:
// a 16-lane group whose lane 4 r + q points at row r, columns 4 q .. 4 q + 3 returns column i of
// those four rows in its lane i).
__device__ __forceinline__ bf16x8 kfrag(const __bf16* tile, int stride, int k0, int col0, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int g = lane / 16, r = (lane % 16) / 4, q = lane % 4;
    const __bf16* p = tile + (k0 + 8 * g + r) * stride + col0 + 4 * q;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * stride));
    const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}
// An MFMA operand contracting over columns k0 .. k0 + 31 of a row-major bf16 LDS tile [row][k]:
// lane (g, i) receives tile[row0 + i][k0 + 8 g + j], j = 0..7 (one 16-byte read).
__device__ __forceinline__ bf16x8 rfrag(const __bf16* tile, int stride, int row0, int k0, int lane) {
    return as_bf16x8(ld16(tile + (row0 + lane % 16) * stride + k0 + 8 * (lane / 16)));
}

template <int N, int P>
__global__ void __launch_bounds__(kBThreads) bwd_states_bf16_kernel(BwdParams prm) {
    using S = BwdBf16Shape<N, P>;
    constexpr int Q = S::Q, PB = S::PB, XS = S::XS, NSB = S::NSB, NTILE = S::NTILE, TPW = S::TPW;
    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen, units = prm.batch * H;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, units);
    if (unit < 0) return;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
    const int nch = prm.seq_off ? (int)((sq.len + kBQ - 1) / kBQ) : prm.nchunks;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, lg = lane / 16, l16 = lane % 16;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Bw = reinterpret_cast<__bf16*>(smem);  // w o B [Q][NSB]
    __bf16* Xs = Bw + Q * NSB;                     // x [Q][XS]
    __shared__ float cum[kBQ];
    __shared__ float e_unused[kBQ], w_s[kBQ];
    const __bf16* xg = static_cast<const __bf16*>(prm.x);
    const __bf16* Bg = static_cast<const __bf16*>(prm.Bm);
    __bf16* ckpt = reinterpret_cast<__bf16*>(prm.ckpt);  // [B,H,nchunks,N,P] bf16

    // H^T in accumulators: tile (pb, nb) holds rows p = 16 pb + 4 lg + i, column n = 16 nb + l16
    f32x4 hs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        hs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wave + kBWaves * j;
        if (tile < NTILE && prm.init) {
            const int pb = tile % PB, nb = tile / PB;
            hs[j] = *reinterpret_cast<const f32x4*>(prm.init + (unit * N + 16 * nb + l16) * P + 16 * pb + 4 * lg);
        }
    }
    ChunkRows<__bf16, Q, N> rb;
    ChunkRows<__bf16, Q, P> rx;
    float rla = 0.f;
    auto load = [&](int c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        rb.load(Bg + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rx.load(xg + ((sq.row0 + t0) * H + h) * P, H * P, len, tid);
        rla = tid < len && tid < Q ? prm.log_a[(sq.row0 + t0 + tid) * H + h] : 0.f;
    };
    if (nch > 0) load(0);
    for (int c = 0; c < nch; ++c) {
        // the checkpoint: the state entering chunk c, four consecutive p per lane
        __bf16* ck = ckpt + (unit * prm.nchunks + c) * (int64_t)N * P;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int pb = tile % PB, nb = tile / PB;
                store4(ck + (16 * nb + l16) * P + 16 * pb + 4 * lg, hs[j][0], hs[j][1], hs[j][2], hs[j][3]);
            }
        }
        chunk_factors_dpp(rla, cum, e_unused, w_s, tid);
        lds_barrier();
        rx.stage_raw(Xs, XS, tid);
        // w o B, rounded once (rows past the end are zeros)
#pragma unroll
        for (int i = 0; i < ChunkRows<__bf16, Q, N>::PT; ++i) {
            constexpr int PER_ROW = ChunkRows<__bf16, Q, N>::PER_ROW, PIECES = ChunkRows<__bf16, Q, N>::PIECES;
            const int u = tid + kBThreads * i, r = u / PER_ROW, cc = (u % PER_ROW) * 8;
            if (u < PIECES) {
                const float wr = w_s[r];
                const bf16x8 bv = as_bf16x8(rb.v[i]);
                bf16x8 o;
#pragma unroll
                for (int k = 0; k < 8; ++k) o[k] = (__bf16)((float)bv[k] * wr);
                *reinterpret_cast<bf16x8*>(Bw + r * NSB + cc) = o;
            }
        }
        const float el = __expf(cum[Q - 1]);
        lds_barrier();
        if (c + 1 < nch) load(c + 1);
        // H^T <- e_last H^T + X^T (w o B): A(p, t) = x[t][p], B(t, n) = (w o B)[t][n]
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int pb = tile % PB, nb = tile / PB;
                hs[j] = mfma_bf16(kfrag(Xs, XS, 0, 16 * pb, lane), kfrag(Bw, NSB, 0, 16 * nb, lane), hs[j] * el);
            }
        }
        lds_barrier();
    }
}

template <int N, int P>
__global__ void __launch_bounds__(kBThreads) bwd_walk_bf16_kernel(BwdParams prm) {
    using S = BwdBf16Shape<N, P>;
    constexpr int Q = S::Q, QF = S::QF, NB = S::NB, PB = S::PB, QB = S::QB;
    constexpr int XS = S::XS, NSB = S::NSB, QSB = S::QSB, NTILE = S::NTILE, TPW = S::TPW;
    static_assert(2 * QB * QB <= kBWaves, "one S o L or DYX tile per wave");
    static_assert(Q * 16 == kBThreads, "row and column sums: 16 threads per row");
    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen, units = prm.batch * H;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, units);
    if (unit < 0) return;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
    const int nch = prm.seq_off ? (int)((sq.len + kBQ - 1) / kBQ) : prm.nchunks;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, lg = lane / 16, l16 = lane % 16;

    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Xb = reinterpret_cast<__bf16*>(smem);  // x [Q][XS]
    __bf16* Yb = Xb + Q * XS;                      // dy [Q][XS]
    __bf16* Bb = Yb + Q * XS;                      // B [Q][NSB]
    __bf16* Cb = Bb + Q * NSB;                     // C [Q][NSB]
    __bf16* Ab = Cb + Q * NSB;                     // S o L [Q][QSB] (rows t, columns s)
    __bf16* Wb = Ab + Q * QSB;                     // L o DYX [Q][QSB]
    __bf16* Hb = Wb + Q * QSB;                     // H [N][XS]
    __bf16* Gb = Hb + N * XS;                      // G [N][XS]
    float* Af = reinterpret_cast<float*>(Gb + N * XS);  // S o L [Q][QF]
    float* Df = Af + Q * QF;                            // DYX [Q][QF]
    float* ev = Df + Q * QF;
    float* wv = ev + Q;
    float* rowM = wv + Q;           // sum_s M_ts
    float* colM = rowM + Q;         // sum_t M_ts
    float* partB = colM + Q;        // [Q][NB]: B_s . (G x_s) over 16-row pieces of n
    float* partC = partB + Q * NB;  // [Q][NB]: C_t . (H dy_t)
    float* red = partC + Q * NB;    // [kBWaves]
    __shared__ float cum[kBQ];

    const __bf16* xg = static_cast<const __bf16*>(prm.x);
    const __bf16* yg = static_cast<const __bf16*>(prm.dy);
    const __bf16* Bg = static_cast<const __bf16*>(prm.Bm);
    const __bf16* Cg = static_cast<const __bf16*>(prm.Cm);
    const __bf16* ckpt = reinterpret_cast<const __bf16*>(prm.ckpt);
    __bf16* dxg = static_cast<__bf16*>(prm.dx);
    const float dskip = prm.D ? prm.D[h] : 0.f;

    // G^T, the gradient of the state leaving the current chunk, in accumulators: tile (pb, nb)
    // holds rows p = 16 pb + 4 lg + i, column n = 16 nb + l16; its bf16 copy in Gb
    f32x4 gs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        gs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wave + kBWaves * j;
        if (tile < NTILE && prm.dfinal) {
            const int pb = tile % PB, nb = tile / PB;
            gs[j] = *reinterpret_cast<const f32x4*>(prm.dfinal + (unit * N + 16 * nb + l16) * P + 16 * pb + 4 * lg);
        }
    }
    auto write_g = [&]() {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int pb = tile % PB, nb = tile / PB;
                store4(Gb + (16 * nb + l16) * XS + 16 * pb + 4 * lg, gs[j][0], gs[j][1], gs[j][2], gs[j][3]);
            }
        }
    };
    write_g();
    float dD_acc = 0.f;

    // the next chunk's inputs, a chunk ahead (chunks run last to first)
    ChunkRows<__bf16, Q, P> rx, ry;
    ChunkRows<__bf16, Q, N> rb, rc;
    ChunkRows<__bf16, N, P> rh;
    float rla = 0.f;
    auto load = [&](int c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        rx.load(xg + ((sq.row0 + t0) * H + h) * P, H * P, len, tid);
        ry.load(yg + ((sq.row0 + t0) * H + h) * P, H * P, len, tid);
        rb.load(Bg + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rc.load(Cg + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rh.load(ckpt + (unit * prm.nchunks + c) * (int64_t)N * P, P, N, tid);
        rla = tid < len && tid < Q ? prm.log_a[(sq.row0 + t0 + tid) * H + h] : 0.f;
    };
    if (nch > 0) load(nch - 1);

    constexpr int JDX = QB * PB, JDB = QB * NB;  // phase-3 jobs: dx tiles; dB and dC tiles (one job each)
    for (int c = nch - 1; c >= 0; --c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        // ---- 1. the chunk's x, dy, B, C and entering state into LDS (zeros past the end)
        rx.stage_raw(Xb, XS, tid);
        ry.stage_raw(Yb, XS, tid);
        rb.stage_raw(Bb, NSB, tid);
        rc.stage_raw(Cb, NSB, tid);
        rh.stage_raw(Hb, XS, tid);
#pragma unroll
        for (int i = 0; i < ChunkRows<__bf16, Q, P>::PT; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) dD_acc += rx.elem(i, j) * ry.elem(i, j);
        chunk_factors_dpp(rla, cum, ev, wv, tid);
        lds_barrier();
        if (c > 0) load(c - 1);

        // ---- 2. S o L (waves 0 .. 3) and DYX, L o DYX (waves 4 .. 7), one 16 x 16 tile (tb, sb) each:
        //         rows t, columns s
        {
            const int job = wave % (QB * QB), tb = job / QB, sb = job % QB;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (wave < QB * QB) {
#pragma unroll
                for (int k = 0; k < N / 32; ++k)
                    v = mfma_bf16(rfrag(Cb, NSB, 16 * tb, 32 * k, lane), rfrag(Bb, NSB, 16 * sb, 32 * k, lane), v);
            } else {
#pragma unroll
                for (int k = 0; k < P / 32; ++k)
                    v = mfma_bf16(rfrag(Yb, XS, 16 * tb, 32 * k, lane), rfrag(Xb, XS, 16 * sb, 32 * k, lane), v);
            }
            const int s = 16 * sb + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * lg + i;
                const float L = s <= t ? __expf(cum[t] - cum[s]) : 0.f;
                if (wave < QB * QB) {
                    Af[t * QF + s] = v[i] * L;
                    Ab[t * QSB + s] = (__bf16)(v[i] * L);
                } else {
                    Df[t * QF + s] = v[i];
                    Wb[t * QSB + s] = (__bf16)(v[i] * L);
                }
            }
        }
        lds_barrier();

        // ---- 3. row and column sums of M = (S o L) o DYX (16 threads per row or column); dx, dB, dC
        //         and the state terms of dcum, tiles dealt to the waves
        {
            const int r = tid / 16, j = tid % 16;
            float rs = 0.f, cs = 0.f;
#pragma unroll
            for (int k = 2 * j; k < 2 * j + 2; ++k) {
                rs += Af[r * QF + k] * Df[r * QF + k];
                cs += Af[k * QF + r] * Df[k * QF + r];
            }
            rs = row16_sum(rs);
            cs = row16_sum(cs);
            if (j == 0) {
                rowM[r] = rs;
                colM[r] = cs;
            }
        }
        // This wave's jobs: dx tiles (wave + kBWaves u), then dB and dC tiles of the same rows and
        // columns together (dB rows s, dC rows t, both columns n), each job's products straight-line
        // and its epilogue right after them.
        {
            constexpr int UX = (JDX + kBWaves - 1) / kBWaves, UB = (JDB + kBWaves - 1) / kBWaves;
#pragma unroll
            for (int u = 0; u < UX; ++u) {
                // dx^T (rows p, columns s) = dY^T (S o L) + w_s G^T B_s + D dy
                const int job = min(wave + kBWaves * u, JDX - 1), sb = job % QB, pb = job / QB;
                const f32x4 xa = mfma_bf16(kfrag(Yb, XS, 0, 16 * pb, lane), kfrag(Ab, QSB, 0, 16 * sb, lane),
                                           f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 xg = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < N / 32; ++k)
                    xg = mfma_bf16(kfrag(Gb, XS, 32 * k, 16 * pb, lane), rfrag(Bb, NSB, 16 * sb, 32 * k, lane), xg);
                const int s = 16 * sb + l16, p0 = 16 * pb + 4 * lg;
                if (wave + kBWaves * u < JDX && s < len) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    const bf16x4 dy4 = *reinterpret_cast<const bf16x4*>(Yb + s * XS + p0);
                    const float ws_ = wv[s];
                    float o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = xa[i] + ws_ * xg[i] + dskip * (float)dy4[i];
                    store4(dxg + ((sq.row0 + t0 + s) * H + h) * P + p0, o[0], o[1], o[2], o[3]);
                }
            }
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                // dB (rows s, columns n) = (L o DYX)^T C + w_s (G x_s) and dC (rows t, columns n) =
                // (L o DYX) B + e_t (H dy_t): one instruction's atomic adds cover 4 rows x 64
                // contiguous bytes (the heads of a group add into the same rows)
                const int job = min(wave + kBWaves * u, JDB - 1), sb = job % QB, nb = job / QB;
                const f32x4 ba = mfma_bf16(kfrag(Wb, QSB, 0, 16 * sb, lane), kfrag(Cb, NSB, 0, 16 * nb, lane),
                                           f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 bg = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < P / 32; ++k)
                    bg = mfma_bf16(rfrag(Xb, XS, 16 * sb, 32 * k, lane), rfrag(Gb, XS, 16 * nb, 32 * k, lane), bg);
                const f32x4 ca = mfma_bf16(rfrag(Wb, QSB, 16 * sb, 0, lane), kfrag(Bb, NSB, 0, 16 * nb, lane),
                                           f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 ch = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < P / 32; ++k)
                    ch = mfma_bf16(rfrag(Yb, XS, 16 * sb, 32 * k, lane), rfrag(Hb, XS, 16 * nb, 32 * k, lane), ch);
                if (wave + kBWaves * u < JDB) {
                    const int n = 16 * nb + l16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = 16 * sb + 4 * lg + i;
                        if (s < len) {
                            atomicAdd(prm.dB + ((sq.row0 + t0 + s) * G + g) * N + n, ba[i] + wv[s] * bg[i]);
                            atomicAdd(prm.dC + ((sq.row0 + t0 + s) * G + g) * N + n, ca[i] + ev[s] * ch[i]);
                        }
                        // B_s . (G x_s) and C_t . (H dy_t) over this tile's 16 columns of n
                        const float pb_ = row16_sum((float)Bb[s * NSB + n] * bg[i]);
                        const float pc_ = row16_sum((float)Cb[s * NSB + n] * ch[i]);
                        if (l16 == 0) {
                            partB[s * NB + nb] = pb_;
                            partC[s * NB + nb] = pc_;
                        }
                    }
                }
            }
        }
        // <G, H> over this wave's tiles
        float gh = 0.f;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int pb = tile % PB, nb = tile / PB;
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                const bf16x4 h4 = *reinterpret_cast<const bf16x4*>(Hb + (16 * nb + l16) * XS + 16 * pb + 4 * lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) gh += gs[j][i] * (float)h4[i];
            }
        }
        gh = wave_sum_dpp(gh);
        if (lane == 0) red[wave] = gh;
        lds_barrier();

        // ---- 4. dcum and dlog a as its reverse running sum (wave 0); the gradient entering the
        //         chunk, G^T <- e_last G^T + dY^T (e o C) (every wave)
        const float el = ev[Q - 1];
        if (tid < kWave) {
            float d = 0.f, wpb = 0.f;
            if (tid < Q) {
                const int t = tid;
                float pb_ = 0.f, pc_ = 0.f;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    pb_ += partB[t * NB + nb];
                    pc_ += partC[t * NB + nb];
                }
                d = rowM[t] - colM[t] + ev[t] * pc_ - wv[t] * pb_;
                wpb = wv[t] * pb_;
            }
            // the last token's term: e_last <G, H> + sum_s w_s B_s . (G x_s)
            const float wsum = wave_sum_dpp(wpb);
            if (tid == Q - 1) {
                float ghs = 0.f;
#pragma unroll
                for (int k = 0; k < kBWaves; ++k) ghs += red[k];
                d += el * ghs + wsum;
            }
            // reverse inclusive running sum over t: inside each 16-lane row by DPP left shifts, then
            // row 1's total into row 0
            float r = tid < Q ? d : 0.f;
            r += bdpp<0x101>(r);  // row_shl:1
            r += bdpp<0x102>(r);  // row_shl:2
            r += bdpp<0x104>(r);  // row_shl:4
            r += bdpp<0x108>(r);  // row_shl:8
            const float row1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), 16));
            r += tid < 16 ? row1 : 0.f;
            if (tid < len) prm.dlog_a[(sq.row0 + t0 + tid) * H + h] = r;
        }
        {
            // e_t for the operand's tokens 8 lg + j
            const f32x4 e0 = *reinterpret_cast<const f32x4*>(ev + 8 * lg);
            const f32x4 e1 = *reinterpret_cast<const f32x4*>(ev + 8 * lg + 4);
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int tile = wave + kBWaves * j;
                if (tile < NTILE) {
                    const int pb = tile % PB, nb = tile / PB;
                    const bf16x8 cv = kfrag(Cb, NSB, 0, 16 * nb, lane);
                    bf16x8 ec;
#pragma unroll
                    for (int k = 0; k < 8; ++k) ec[k] = (__bf16)((float)cv[k] * (k < 4 ? e0[k] : e1[k - 4]));
                    gs[j] = mfma_bf16(kfrag(Yb, XS, 0, 16 * pb, lane), ec, gs[j] * el);
                }
            }
        }
        lds_barrier();  // every read of Gb, Hb and the chunk tiles above is done
        write_g();
    }
    lds_barrier();
    if (prm.dinit) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kBWaves * j;
            if (tile < NTILE) {
                const int pb = tile % PB, nb = tile / PB;
                *reinterpret_cast<f32x4*>(prm.dinit + (unit * N + 16 * nb + l16) * P + 16 * pb + 4 * lg) = gs[j];
            }
        }
    }
    // dy . x over the unit, for dD
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dD_acc += __shfl_xor(dD_acc, off, kWave);
    if (lane == 0) red[wave] = dD_acc;
    lds_barrier();
    if (tid == 0) {
        float s = 0.f;
        for (int k = 0; k < kBWaves; ++k) s += red[k];
        prm.dD_part[unit] = s;
    }
}

// ---------------------------------------------------------------------------------------
// Diagonal decay (one log a per state dimension n).  The same chain rule, with per-(t, n) running
// sums cum_tn, e_tn = exp(cum_tn), w_sn = exp(cum_last,n - cum_sn), L_tsn = exp(cum_tn - cum_sn):
//   A_ts    = sum_n C_tn B_sn L_tsn                      (the scores, decay inside the sum)
//   dx_s    = sum_t A_ts dy_t + sum_n w_sn B_sn G_n + D dy_s
//   dB_sn  += sum_t L_tsn DYX_ts C_tn + w_sn (G x_s)_n
//   dC_tn  += sum_s L_tsn DYX_ts B_sn + e_tn (H dy_t)_n
//   dcum_tn = sum_s M_tsn - sum_t' M_t'tn + e_tn C_tn (H dy_t)_n - w_tn B_tn (G x_t)_n
//             + [t = last] (e_last,n <G_n, H_n> + sum_s w_sn B_sn (G x_s)_n),  M_tsn = C_tn B_sn L_tsn DYX_ts
// with H the state entering the chunk and G the gradient of the state at its end.  Both are chains
// over the chunks, H_{c+1} = e_last,n H_c + sum_s w_sn B_sn x_s^T and G_{c-1} = e_last,n G_c +
// sum_t e_tn C_tn dy_t^T, of the same associative form as the forward's state passing.  So the pass
// runs every chunk at once: a local kernel per (unit, chunk) forms the intra-chunk terms and the
// two local sums; a scan per state element chains the sums into H and G in place; a second kernel
// per (unit, chunk) adds the terms that need H and G.
// Over a chunk of fast-decaying dimensions exp(cum_tn - cum_sn) spans more than fp32 can hold in any
// pair of factors, so the intra-chunk sums run on the vector units with an exact exp per (t, s, n);
// the carried-state terms stay on the matrix cores with the per-(t, n) factor folded into an operand.
template <int N, int P, typename CT>
struct BwdDiagShape {
    // NC: row stride of the [Q][N] arrays (padded so that rows fall on different LDS banks)
    static constexpr int Q = kBQ, QS = Q + 1, NS = N + 1, PS = P + 1, NC = N + 1;
    static constexpr int NB = N / 16, PB = P / 16, QB = Q / 16;
    static constexpr size_t cum_bytes = ((size_t)Q * NC * sizeof(CT) + 15) / 16 * 16;
    // local LDS: cum [Q][NC] of CT; floats: X, dY [Q][PS]; B, C [Q][NS]; A, DYX [Q][QS]; w, e
    // [Q][NC]; C o f, B o g [16][NC]; e_last [N]; partial sums [kWaves]
    static constexpr size_t local_lds =
        cum_bytes + ((size_t)2 * Q * PS + 2 * Q * NS + 2 * Q * QS + 2 * Q * NC + 32 * NC + N + kWaves) * 4;
    // state-terms LDS: cum [Q][NC] of CT; floats: X, dY [Q][PS]; B, C [Q][NS]; e, w, dcum [Q][NC];
    // H, G [N][PS]; e_last, <G_n, H_n> [N]; partial last-token sums [QB][N]
    static constexpr size_t terms_lds =
        cum_bytes + ((size_t)2 * Q * PS + 2 * Q * NS + 3 * Q * NC + 2 * N * PS + 2 * N + QB * N) * 4;
};

// The diagonal path's running sums: fp64 natural-log units with the library exp for fp32 inputs;
// log2 units with the hardware exp2 (v_exp_f32) for bf16 inputs, one instruction per factor.
template <typename CT> struct DiagExp;
template <> struct DiagExp<double> {
    static constexpr double kScale = 1.0;
    __device__ static double ex(double v) { return exp(v); }
};
template <> struct DiagExp<float> {
    static constexpr float kScale = 1.4426950408889634f;
    __device__ static float ex(float v) { return __builtin_amdgcn_exp2f(v); }
};

// Per-dimension running sums of one chunk's log a (la [Q][N], 0 past the end), by threads n < N:
// cum, e, w (may be la itself: each thread overwrites only its own column, after reading all of it)
// and e_last.  The column is read into registers first, so the LDS loads run back to back.
template <int N, typename CT>
__device__ __forceinline__ void diag_chunk_factors(const float* la, CT* cum, float* e, float* w, float* el, int tid) {
    constexpr int NC = N + 1;  // (row stride of every [Q][N] array)
    if (tid < N) {
        const int n = tid;
        CT c[kBQ];
        CT run = 0;
#pragma unroll
        for (int t = 0; t < kBQ; ++t) {
            run += (CT)la[t * NC + n] * DiagExp<CT>::kScale;
            c[t] = run;
        }
#pragma unroll
        for (int t = 0; t < kBQ; ++t) {
            cum[t * NC + n] = c[t];
            e[t * NC + n] = (float)DiagExp<CT>::ex(c[t]);
            w[t * NC + n] = (float)DiagExp<CT>::ex(run - c[t]);
        }
        el[n] = (float)DiagExp<CT>::ex(run);
    }
}

// The local kernel of the diagonal backward, one workgroup per (batch, head, chunk).  For the
// chunk's rows it writes dx_intra = sum_t A_ts dy_t, intra dB and dC, and dcum_intra = sum_s M_tsn -
// sum_t' M_t'tn; for the chunk, its local state sum S = sum_s w_sn B_sn x_s^T (into the checkpoint
// slot), its local gradient sum U = sum_t e_tn C_tn dy_t^T (into the gradient slot), e_last and
// sum x . dy.  The grid also clears dB and dC, which the state-terms kernel accumulates into.
//
// The intra-chunk sums over pairs t >= s split by 16-token blocks.  Across the two blocks (t in the
// second, s in the first) L_tsn = f_tn g_sn with f_tn = exp(cum_tn - cum_15,n) and g_sn =
// exp(cum_15,n - cum_sn), both at most 1 because log a <= 0: those terms are products on the matrix
// cores, (C o f)(B o g)^T for A, DYX^T (C o f) for dB and DYX (B o g) for dC.  Inside a block each
// L_tsn is one exact exp, used once for A (a thread per pair, summing over n) and once for dB and dC
// together (a thread per (block, n), summing over the block's pairs).
template <typename T, int N, int P>
__global__ void __launch_bounds__(kThreads) bwd_local_diag_kernel(BwdParams prm) {
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    using S = BwdDiagShape<N, P, CT>;
    constexpr int Q = S::Q, QS = S::QS, NS = S::NS, PS = S::PS, NB = S::NB, PB = S::PB, QB = S::QB, NC = S::NC;
    static_assert(QB == 2 && QB * QB == kWaves, "two 16-token blocks; one DYX tile per wave");
    static_assert(N <= kWave, "one lane per state dim in the exact block sums");
    constexpr int kPairs = 16 * 17 / 2;  // pairs t >= s inside one block
    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen, units = prm.batch * H;
    const int64_t nch = prm.nchunks;
    {
        const int64_t nbc = (prm.seq_off ? prm.total : prm.batch * Tn) * G * N, stride = (int64_t)gridDim.x * kThreads;
        for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nbc; i += stride) {
            prm.dB[i] = 0.f;
            prm.dC[i] = 0.f;
        }
    }
    const int64_t work = xcd_work_index(blockIdx.x, prm.per_xcd_intra, units * nch);
    if (work < 0) return;
    const int64_t unit = work / nch;
    const int c = (int)(work % nch);
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, lg = lane / 16, l16 = lane % 16;
    const int r = lane % 16, gq = lane / 16;
    const int64_t t0 = (int64_t)c * Q;
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
    if (t0 >= sq.len) {
        // (a packed sequence shorter than seqlen: no such chunk; nothing for dD from it)
        if (threadIdx.x == 0) prm.dD_part[unit * nch + c] = 0.f;
        return;
    }
    const int len = (int)min((int64_t)Q, sq.len - t0);

    extern __shared__ __align__(16) unsigned char smem[];
    CT* cum = reinterpret_cast<CT*>(smem);                    // [Q][NC]
    float* Xs = reinterpret_cast<float*>(smem + S::cum_bytes);  // [Q][PS]
    float* Ys = Xs + Q * PS;                                  // dy [Q][PS]
    float* Bs = Ys + Q * PS;                                  // [Q][NS]
    float* Cs = Bs + Q * NS;                                  // [Q][NS]
    float* Am = Cs + Q * NS;                                  // A [Q][QS]
    float* Dm = Am + Q * QS;                                  // DYX [Q][QS]
    float* Wv = Dm + Q * QS;                                  // log a, then w, then the in-block dB [Q][NC]
    float* Ev = Wv + Q * NC;                                  // e, then the in-block dC [Q][NC]
    float* Cf = Ev + Q * NC;                                  // C_tn f_tn, t = 16 + row [16][NC]
    float* Bg = Cf + 16 * NC;                                 // B_sn g_sn [16][NC]
    float* el = Bg + 16 * NC;                                 // e_last [N]
    float* red = el + N;                                      // [kWaves]

    // the chunk's rows into LDS in 16-byte pieces, every load issued first (zeros past the end);
    // sum x . dy on the way
    float xdy = 0.f;
    {
        const int64_t rowx = (sq.row0 + t0) * H + h, rowb = (sq.row0 + t0) * G + g;
        ChunkRows<T, Q, P, kThreads> rx, ry;
        ChunkRows<T, Q, N, kThreads> rb, rc;
        ChunkRows<float, Q, N, kThreads> rl;
        rx.load(static_cast<const T*>(prm.x) + rowx * P, H * P, len, tid);
        ry.load(static_cast<const T*>(prm.dy) + rowx * P, H * P, len, tid);
        rb.load(static_cast<const T*>(prm.Bm) + rowb * N, G * N, len, tid);
        rc.load(static_cast<const T*>(prm.Cm) + rowb * N, G * N, len, tid);
        rl.load(prm.log_a + rowx * N, H * N, len, tid);
        rx.stage(Xs, PS, tid);
        ry.stage(Ys, PS, tid);
        rb.stage(Bs, NS, tid);
        rc.stage(Cs, NS, tid);
        rl.stage(Wv, NC, tid);
        using RX = ChunkRows<T, Q, P, kThreads>;
#pragma unroll
        for (int i = 0; i < RX::PT; ++i)
#pragma unroll
            for (int j = 0; j < RX::VE; ++j) xdy += rx.elem(i, j) * ry.elem(i, j);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) xdy += __shfl_xor(xdy, off, kWave);
    if (lane == 0) red[wave] = xdy;
    lds_barrier();
    diag_chunk_factors<N, CT>(Wv, cum, Ev, Wv, el, tid);
    {
        const int tb = wave / QB, sb = wave % QB;
        const f32x4 v = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Ys + 16 * tb * PS, PS, 1, Xs + 16 * sb * PS, 1, PS, P,
                                 lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) Dm[(16 * tb + 4 * lg + i) * QS + 16 * sb + l16] = v[i];
    }
    lds_barrier();

    // ---- 1. e_last and sum x . dy out; the local sums S = (w o B)^T X and U = (e o C)^T dY; the
    //         cross-block operands C o f and B o g
    const int64_t row0 = (sq.row0 + t0) * H + h;
    if (tid < N) prm.elw[(unit * nch + c) * N + tid] = el[tid];
    if (tid == 0) prm.dD_part[unit * nch + c] = (red[0] + red[1]) + (red[2] + red[3]);
    {
        float* Sg = prm.ckpt + (unit * nch + c) * (int64_t)N * P;
        float* Ug = prm.gst + (unit * nch + c) * (int64_t)N * P;
        for (int tile = wave; tile < 2 * NB * PB; tile += kWaves) {
            const bool isU = tile >= NB * PB;
            const int tt = isU ? tile - NB * PB : tile, nb = tt / PB, pb = tt % PB;
            const float* F = isU ? Ev : Wv;
            const float* V = isU ? Cs : Bs;
            const float* R = isU ? Ys : Xs;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < Q; k += 4) {
                const int s = k + gq, n = 16 * nb + r;
                acc = mfma_f32(F[s * NC + n] * V[s * NS + n], R[s * PS + 16 * pb + r], acc);
            }
            float* out = isU ? Ug : Sg;
#pragma unroll
            for (int i = 0; i < 4; ++i) out[(16 * nb + 4 * lg + i) * P + 16 * pb + l16] = acc[i];
        }
    }
    for (int i = tid; i < 16 * N; i += kThreads) {
        const int j = i / N, n = i % N;
        const CT ref = cum[15 * NC + n];
        Cf[j * NC + n] = Cs[(16 + j) * NS + n] * (float)DiagExp<CT>::ex(cum[(16 + j) * NC + n] - ref);
        Bg[j * NC + n] = Bs[j * NS + n] * (float)DiagExp<CT>::ex(ref - cum[j * NC + n]);
    }
    lds_barrier();

    // ---- 2. waves 0, 1: the in-block dB, dC of block `wave` for dim `lane` (into Wv, Ev);
    //         waves 2, 3: A, in-block pairs exact, the cross block on the matrix cores, zeros above
    if (wave < 2) {
        const int o = 16 * wave, n = lane;
        if (n < N) {
            float cv[16], bv[16], db[16], dc[16];
            CT cm[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                cv[j] = Cs[(o + j) * NS + n];
                bv[j] = Bs[(o + j) * NS + n];
                cm[j] = cum[(o + j) * NC + n];
                db[j] = 0.f;
                dc[j] = 0.f;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t)
#pragma unroll
                for (int s2 = 0; s2 <= t; ++s2) {
                    const float d = Dm[(o + t) * QS + o + s2] * (float)DiagExp<CT>::ex(cm[t] - cm[s2]);
                    db[s2] += d * cv[t];
                    dc[t] += d * bv[s2];
                }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                Wv[(o + j) * NC + n] = db[j];
                Ev[(o + j) * NC + n] = dc[j];
            }
        }
    } else {
        const int u = tid - 2 * kWave;  // 0 .. 127
        if (wave == 2) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k = 0; k < N; k += 4) acc = mfma_f32(Cf[r * NC + k + gq], Bg[r * NC + k + gq], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Am[(16 + 4 * lg + i) * QS + l16] = acc[i];
                Am[(4 * lg + i) * QS + 16 + l16] = 0.f;
            }
        }
        for (int z = u; z < 2 * 256; z += 2 * kWave) {
            const int blk = z / 256, i = (z % 256) / 16, j = z % 16;
            if (j > i) Am[(16 * blk + i) * QS + 16 * blk + j] = 0.f;
        }
        for (int pi = u; pi < 2 * kPairs; pi += 2 * kWave) {
            const int blk = pi / kPairs, pr = pi % kPairs;
            int i = (int)((sqrtf(8.f * pr + 1.f) - 1.f) * 0.5f);
            if ((i + 1) * (i + 2) / 2 <= pr) ++i;
            if (i * (i + 1) / 2 > pr) --i;
            const int j = pr - i * (i + 1) / 2;
            const int t = 16 * blk + i, s2 = 16 * blk + j;
            float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int n = 0; n < N; n += 4)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    a[v] += Cs[t * NS + n + v] * Bs[s2 * NS + n + v] *
                            (float)DiagExp<CT>::ex(cum[t * NC + n + v] - cum[s2 * NC + n + v]);
            Am[t * QS + s2] = (a[0] + a[1]) + (a[2] + a[3]);
        }
    }
    lds_barrier();

    // ---- 3. the cross-block dB (rows s < 16) and dC (rows t >= 16) on the matrix cores, added to the
    //         in-block sums; every (q, n) written once, with dcum_intra = C dC - B dB; then dx_intra
    for (int tile = wave; tile < 2 * NB + QB * PB; tile += kWaves) {
        if (tile < 2 * NB) {
            const bool isB = tile < NB;
            const int nb = isB ? tile : tile - NB, n = 16 * nb + l16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 16; k += 4) {
                // dB: A(s, t') = DYX[16 + t'][s], B(t', n) = Cf[t'][n];  dC: A(t', s) = DYX[16 + t'][s], B(s, n) = Bg[s][n]
                const float av = isB ? Dm[(16 + k + gq) * QS + r] : Dm[(16 + r) * QS + k + gq];
                const float bv = isB ? Cf[(k + gq) * NC + n - l16 + r] : Bg[(k + gq) * NC + n - l16 + r];
                acc = mfma_f32(av, bv, acc);
            }
            const CT ref = cum[15 * NC + n];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = (isB ? 0 : 16) + 4 * lg + i;
                float dbv = Wv[q * NC + n], dcv = Ev[q * NC + n];
                if (isB)
                    dbv += acc[i] * (float)DiagExp<CT>::ex(ref - cum[q * NC + n]);
                else
                    dcv += acc[i] * (float)DiagExp<CT>::ex(cum[q * NC + n] - ref);
                if (q < len) {
                    const int64_t o = (row0 + (int64_t)q * H) * N + n;
                    prm.dBi[o] = dbv;
                    prm.dCi[o] = dcv;
                    prm.dcumi[o] = Cs[q * NS + n] * dcv - Bs[q * NS + n] * dbv;
                }
            }
        } else {
            // dx_intra = sum_t A_ts dy_t: A(s, t) = Am[t][s]
            const int tt = tile - 2 * NB, sb = tt / PB, pb = tt % PB;
            const f32x4 acc = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Am + 16 * sb, 1, QS, Ys + 16 * pb, PS, 1, Q, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s2 = 16 * sb + 4 * lg + i;
                if (s2 < len) prm.dxi[(row0 + (int64_t)s2 * H) * P + 16 * pb + l16] = acc[i];
            }
        }
    }
}

// The chains over the chunks, in place, one thread per (batch, head, state element) and direction:
// the checkpoint slots hold S_c on entry and H_c (the state entering chunk c) on exit, from
// H_0 = init; the gradient slots hold U_c on entry and G_c (the gradient of the state at the end of
// chunk c) on exit, from dfinal; dinit = e_last,0 G_0 + U_0.  Loads go 32 chunks at a time.
template <int N, int P>
__global__ void __launch_bounds__(kThreads) bwd_scan_diag_kernel(BwdParams prm) {
    constexpr int64_t per = (int64_t)N * P;
    constexpr int kB = 32;
    const int64_t units = prm.batch * prm.nheads;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= 2 * units * per) return;
    const bool fwd = i < units * per;
    const int64_t j = fwd ? i : i - units * per;
    const int64_t unit = j / per, e = j % per, n = e / P;
    const int nch = prm.nchunks;  // (the slots' stride)
    // (a packed sequence: its own chunks)
    const int ncb = prm.seq_off
                        ? (int)((seq_span(prm.seq_off, unit / prm.nheads, prm.seqlen, prm.total).len + kBQ - 1) / kBQ)
                        : nch;
    const float* el = prm.elw + unit * nch * N + n;
    float* slot = (fwd ? prm.ckpt : prm.gst) + unit * nch * per + e;
    const float* start = fwd ? prm.init : prm.dfinal;
    float v = start ? start[unit * per + e] : 0.f;
    for (int k0 = 0; k0 < ncb; k0 += kB) {
        float s[kB], a[kB];
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            const int c = fwd ? k0 + k : ncb - 1 - k0 - k;
            if (k0 + k < ncb) {
                s[k] = slot[c * per];
                a[k] = el[c * N];
            }
        }
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            const int c = fwd ? k0 + k : ncb - 1 - k0 - k;
            if (k0 + k < ncb) {
                slot[c * per] = v;
                v = a[k] * v + s[k];
            }
        }
    }
    if (!fwd && prm.dinit) prm.dinit[unit * per + e] = v;
}

// The state-terms kernel of the diagonal backward: with each chunk's H and G from the scan and its
// intra-chunk terms from the local kernel, the dx, dB, dC and dlog a of the chunk's rows (dB and dC
// accumulated over the heads of a group).  Persistent: the workgroups of one XCD walk a contiguous
// range of (batch, head, chunk) items, each loading the next item's rows while it works on the
// current one.
template <typename T, int N, int P>
__global__ void __launch_bounds__(kBThreads) bwd_terms_diag_kernel(BwdParams prm) {
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    using S = BwdDiagShape<N, P, CT>;
    constexpr int Q = S::Q, NS = S::NS, PS = S::PS, NB = S::NB, PB = S::PB, QB = S::QB, NC = S::NC;
    static_assert(QB * PB <= kBWaves && QB * NB <= kBWaves, "at most one dx and one dB/dC tile per wave");
    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen, units = prm.batch * H;
    const int64_t nch = prm.nchunks, items = units * nch;
    const int64_t xcd = blockIdx.x % 8, wg_per_xcd = gridDim.x / 8;
    const int64_t first = xcd * prm.per_xcd_intra, last = min(first + prm.per_xcd_intra, items);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, lg = lane / 16, l16 = lane % 16;
    const int r = lane % 16, gq = lane / 16;

    extern __shared__ __align__(16) unsigned char smem[];
    CT* cum = reinterpret_cast<CT*>(smem);                    // [Q][NC]
    float* Xs = reinterpret_cast<float*>(smem + S::cum_bytes);  // [Q][PS]
    float* Ys = Xs + Q * PS;                                  // dy [Q][PS]
    float* Bs = Ys + Q * PS;                                  // [Q][NS]
    float* Cs = Bs + Q * NS;                                  // [Q][NS]
    float* Ev = Cs + Q * NS;                                  // e [Q][NC]
    float* Wv = Ev + Q * NC;                                  // log a, then w [Q][NC]
    float* dcum = Wv + Q * NC;                                // [Q][NC]
    float* Hs = dcum + Q * NC;                                // H [N][PS]
    float* Gs = Hs + N * PS;                                  // G [N][PS]
    float* el = Gs + N * PS;                                  // e_last [N]
    float* ghn = el + N;                                      // <G_n, H_n> [N]
    float* partL = ghn + N;                                   // [QB][N]: sum_s w_sn B_sn (G x_s)_n per 16 rows

    ChunkRows<T, Q, P> rx, ry;
    ChunkRows<T, Q, N> rb, rc;
    ChunkRows<float, N, P> rh, rg;
    ChunkRows<float, Q, N> rl, rm;
    float dxb[4], dbb[4], dcb[4];
    // every input of item w into registers (this wave's intra-chunk dx, dB and dC elements too)
    auto load = [&](int64_t w) {
        const int64_t unit = w / nch, b = unit / H, h = unit % H, g = h / (H / G);
        const int c = (int)(w % nch);
        const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
        const int64_t t0 = (int64_t)c * Q, row0 = (sq.row0 + t0) * H + h;
        // (rows past a packed sequence's end are neither read nor written: len <= 0 masks them)
        const int len = (int)min((int64_t)Q, sq.len - t0);
        rx.load(static_cast<const T*>(prm.x) + row0 * P, H * P, len, tid);
        ry.load(static_cast<const T*>(prm.dy) + row0 * P, H * P, len, tid);
        rb.load(static_cast<const T*>(prm.Bm) + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rc.load(static_cast<const T*>(prm.Cm) + ((sq.row0 + t0) * G + g) * N, G * N, len, tid);
        rh.load(prm.ckpt + w * (int64_t)N * P, P, N, tid);
        rg.load(prm.gst + w * (int64_t)N * P, P, N, tid);
        rl.load(prm.log_a + row0 * N, H * N, len, tid);
        rm.load(prm.dcumi + row0 * N, H * N, len, tid);
        if (wave < QB * PB) {
            const int sb = wave / PB, p = 16 * (wave % PB) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s2 = 16 * sb + 4 * lg + i;
                dxb[i] = s2 < len ? prm.dxi[(row0 + (int64_t)s2 * H) * P + p] : 0.f;
            }
        }
        if (wave < QB * NB) {
            const int qb = wave / NB, n = 16 * (wave % NB) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = 16 * qb + 4 * lg + i;
                const int64_t o = (row0 + (int64_t)q * H) * N + n;
                dbb[i] = q < len ? prm.dBi[o] : 0.f;
                dcb[i] = q < len ? prm.dCi[o] : 0.f;
            }
        }
    };
    int64_t w = first + blockIdx.x / 8;
    if (w < last) load(w);
    T* dxg = static_cast<T*>(prm.dx);
    for (; w < last; w += wg_per_xcd) {
        const int64_t unit = w / nch, b = unit / H, h = unit % H, g = h / (H / G);
        const int c = (int)(w % nch);
        const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
        const int64_t t0 = (int64_t)c * Q, row0 = (sq.row0 + t0) * H + h;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        const float dskip = prm.D ? prm.D[h] : 0.f;
        lds_barrier();  // the previous item is done with every LDS array
        rx.stage(Xs, PS, tid);
        ry.stage(Ys, PS, tid);
        rb.stage(Bs, NS, tid);
        rc.stage(Cs, NS, tid);
        rh.stage(Hs, PS, tid);
        rg.stage(Gs, PS, tid);
        rl.stage(Wv, NC, tid);
        rm.stage(dcum, NC, tid);
        float cxb[4], cbb[4], ccb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cxb[i] = dxb[i];
            cbb[i] = dbb[i];
            ccb[i] = dcb[i];
        }
        lds_barrier();
        if (w + wg_per_xcd < last) load(w + wg_per_xcd);
        if (len <= 0) continue;  // (a packed sequence shorter than seqlen: no such chunk)
        diag_chunk_factors<N, CT>(Wv, cum, Ev, Wv, el, tid);
        if (tid >= kBThreads - N) {
            const int n = tid - (kBThreads - N);
            float acc = 0.f;
#pragma unroll 8
            for (int p = 0; p < P; ++p) acc += Gs[n * PS + p] * Hs[n * PS + p];
            ghn[n] = acc;
        }
        lds_barrier();

        // dx = dx_intra + sum_n w_sn B_sn G_np + D dy_s
        if (wave < QB * PB) {
            const int sb = wave / PB, pb = wave % PB, p = 16 * pb + l16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k = 0; k < N; k += 4) {
                const int s2 = 16 * sb + r, n = k + gq;
                acc = mfma_f32(Wv[s2 * NC + n] * Bs[s2 * NS + n], Gs[n * PS + 16 * pb + r], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s2 = 16 * sb + 4 * lg + i;
                if (s2 < len)
                    dxg[(row0 + (int64_t)s2 * H) * P + p] = from_f32<T>(cxb[i] + acc[i] + dskip * Ys[s2 * PS + p]);
            }
        }
        // dB, dC out; dcum's state terms
        if (wave < QB * NB) {
            const int qb = wave / NB, nb = wave % NB, n = 16 * nb + l16;
            const f32x4 gx = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Xs + 16 * qb * PS, PS, 1, Gs + 16 * nb * PS, 1, PS,
                                      P, lane);
            const f32x4 hd = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, Ys + 16 * qb * PS, PS, 1, Hs + 16 * nb * PS, 1, PS,
                                      P, lane);
            float lastp = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = 16 * qb + 4 * lg + i;
                const float wb = Wv[q * NC + n] * Bs[q * NS + n] * gx[i];
                const float ec = Ev[q * NC + n] * Cs[q * NS + n] * hd[i];
                if (q < len) {
                    atomicAdd(prm.dB + ((sq.row0 + t0 + q) * G + g) * N + n, cbb[i] + Wv[q * NC + n] * gx[i]);
                    atomicAdd(prm.dC + ((sq.row0 + t0 + q) * G + g) * N + n, ccb[i] + Ev[q * NC + n] * hd[i]);
                }
                dcum[q * NC + n] += ec - wb;
                lastp += wb;
            }
            lastp += __shfl_xor(lastp, 16, kWave);
            lastp += __shfl_xor(lastp, 32, kWave);
            if (lg == 0) partL[qb * N + n] = lastp;
        }
        lds_barrier();

        // dlog a per dimension: reverse running sum, the last token's term first
        if (tid < N) {
            const int n = tid;
            float last2 = el[n] * ghn[n];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) last2 += partL[qb * N + n];
            float acc = last2;
            for (int t = Q - 1; t >= 0; --t) {
                acc += dcum[t * NC + n];
                if (t < len) prm.dlog_a[(row0 + (int64_t)t * H) * N + n] = acc;
            }
        }
    }
}

// dD[h] = sum over the batch (and for the diagonal path the chunks) of the per-unit sums,
// part[(b H + h) nper + k].  (dB and dC are cleared by zero_kernel on the scalar path, by the local
// kernel on the diagonal one.)
__global__ void __launch_bounds__(kThreads) bwd_reduce_kernel(const float* part, float* dD, int64_t batch, int64_t H,
                                                              int64_t nper) {
    // one workgroup per head
    const int64_t h = blockIdx.x;
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < batch * nper; i += kThreads) s += part[((i / nper) * H + h) * nper + i % nper];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, kWave);
    __shared__ float red[kWaves];
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = s;
    lds_barrier();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int k = 0; k < kWaves; ++k) t += red[k];
        dD[h] = t;
    }
}

__global__ void __launch_bounds__(kThreads) zero_kernel(float* a, int64_t n, float* b2, int64_t n2) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) a[i] = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n2; i += stride) b2[i] = 0.f;
}

template <typename T, int N, int P>
int launch_backward_t(const BackwardLaunch& bl, hipStream_t stream) {
    using S = BwdShape<N, P>;
    using SB = BwdBf16Shape<N, P>;
    // bf16 inputs at the shapes the bf16 kernels cover take them
    constexpr bool kBf16 = std::is_same<T, __bf16>::value && bwd_bf16_shape<N, P>();
    static_assert(S::walk_lds + 1024 <= kMaxLds, "backward walk LDS budget (with its static running sums)");
    static_assert(SB::walk_lds + 1024 <= kMaxLds, "bf16 backward walk LDS budget");
    static bool attr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    if (!attr[dev]) {
        // (the dynamic size the kernel uses, not the whole 160 KiB: its static LDS counts too)
        const void* walk;
        size_t lds;
        if constexpr (kBf16) {
            walk = reinterpret_cast<const void*>(&bwd_walk_bf16_kernel<N, P>);
            lds = SB::walk_lds;
        } else {
            walk = reinterpret_cast<const void*>(&bwd_walk_kernel<T, N, P>);
            lds = S::walk_lds;
        }
        if (hipFuncSetAttribute(walk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return -1;
        attr[dev] = true;
    }
    const int64_t units = bl.p.batch * bl.p.nheads;
    BwdParams p = bl.p;
    p.per_xcd = (units + 7) / 8;
    const int64_t nbc = (bl.p.seq_off ? bl.p.total : bl.p.batch * bl.p.seqlen) * bl.p.ngroups * N;
    int k = 0;
    if (nbc > 0 &&
        !launch_k(bl, k, zero_kernel, dim3((unsigned)std::min<int64_t>((nbc + kThreads - 1) / kThreads, 4096)),
                  dim3(kThreads), 0, stream, p.dB, nbc, p.dC, nbc))
        return -1;
    if (units > 0) {
        if constexpr (kBf16) {
            if (!launch_k(bl, k, bwd_states_bf16_kernel<N, P>, dim3((unsigned)(8 * p.per_xcd)), dim3(kBThreads),
                          SB::states_lds, stream, p))
                return -1;
            if (!launch_k(bl, k, bwd_walk_bf16_kernel<N, P>, dim3((unsigned)(8 * p.per_xcd)), dim3(kBThreads),
                          SB::walk_lds, stream, p))
                return -1;
        } else {
            if (!launch_k(bl, k, bwd_states_kernel<T, N, P>, dim3((unsigned)(8 * p.per_xcd)), dim3(kBThreads),
                          S::states_lds, stream, p))
                return -1;
            if (!launch_k(bl, k, bwd_walk_kernel<T, N, P>, dim3((unsigned)(8 * p.per_xcd)), dim3(kBThreads),
                          S::walk_lds, stream, p))
                return -1;
        }
    }
    if (p.dD && !launch_k(bl, k, bwd_reduce_kernel, dim3((unsigned)bl.p.nheads),
                          dim3(kThreads), 0, stream, (const float*)p.dD_part, p.dD, bl.p.batch, bl.p.nheads,
                          (int64_t)1))
        return -1;
    return 0;
}

// ---------------------------------------------------------------------------------------
// The discretised form's backward (ssd_backward_dt), by the chain rule around the backward pass
// above: with u = dt + bias, Delta = softplus(u), log a = -Delta exp(A_log) and the walk run on
// x_in = Delta x (with the input scale) or x,
//   dx = Delta dx_in (or dx_in) + D dy,   dDelta = -exp(A_log) dlog a + [scale] sum_p dx_in x,
//   ddt = dDelta sigmoid(u),   ddt_bias = sum_{b,t} ddt,   dA_log = sum_{b,t} dlog a log a,
//   dD = sum_{b,t,p} dy x.
// CT (double for fp32 inputs, float for bf16) carries the per-row arithmetic.

// Per (b, t, h) row: its K log a values (K = 1 scalar decay, N diagonal) into la, and with the input
// scale Delta x into xs.
template <typename T>
__global__ void __launch_bounds__(kThreads) disc_rows_kernel(const float* dt, const float* dt_bias, const float* A_log,
                                                             const T* x, float* la, T* xs, int64_t rows, int64_t H,
                                                             int P, int K) {
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (r >= rows) return;
    const int64_t h = r % H;
    const CT u = (CT)dt[r] + (dt_bias ? (CT)dt_bias[h] : (CT)0);
    const CT delta = softplus_ct(u);
    for (int n = 0; n < K; ++n) la[r * K + n] = (float)(-delta * exp((CT)A_log[h * K + n]));
    if (xs)
        for (int p = 0; p < P; ++p) xs[r * P + p] = from_f32<T>((float)(delta * (CT)to_f32(x[r * P + p])));
}

// Per row: dx, ddt, and the row terms of dA_log (dlog a log a, K per row) and dD (dy . x).
template <typename T>
__global__ void __launch_bounds__(kThreads) disc_grad_rows_kernel(const float* dt, const float* dt_bias,
                                                                  const float* A_log, const float* D, const T* x,
                                                                  const T* dy, const T* dxs, const float* la,
                                                                  const float* dla, int scale, T* dx, float* ddt,
                                                                  float* rowA, float* rowD, int64_t rows, int64_t H,
                                                                  int P, int K) {
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (r >= rows) return;
    const int64_t h = r % H;
    const CT u = (CT)dt[r] + (dt_bias ? (CT)dt_bias[h] : (CT)0);
    const CT delta = softplus_ct(u);
    const CT dskip = D ? (CT)D[h] : (CT)0;
    CT xdx = 0, xdy = 0;
    for (int p = 0; p < P; ++p) {
        const CT xv = (CT)to_f32(x[r * P + p]), gv = (CT)to_f32(dxs[r * P + p]), yv = (CT)to_f32(dy[r * P + p]);
        xdx += xv * gv;
        xdy += xv * yv;
        dx[r * P + p] = from_f32<T>((float)((scale ? delta * gv : gv) + dskip * yv));
    }
    CT ddelta = scale ? xdx : (CT)0;
    for (int n = 0; n < K; ++n) {
        const CT dlog = (CT)dla[r * K + n];
        ddelta += -exp((CT)A_log[h * K + n]) * dlog;
        rowA[r * K + n] = (float)(dlog * (CT)la[r * K + n]);
    }
    ddt[r] = (float)(ddelta / (1 + exp(-u)));
    rowD[r] = (float)xdy;
}

// out[h] = sum over the (b, t) rows of head h of v (rows = (b, t) * H + h), one workgroup per head.
__global__ void __launch_bounds__(kThreads) head_sum_kernel(const float* v, float* out, int64_t bt, int64_t H) {
    const int64_t h = blockIdx.x;
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < bt; i += kThreads) s += v[i * H + h];
    __shared__ float red[kThreads];
    red[threadIdx.x] = s;
    lds_barrier();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        lds_barrier();
    }
    if (threadIdx.x == 0) out[h] = red[0];
}

template <typename T, int N, int P>
int launch_backward_diag_t(const BackwardLaunch& bl, hipStream_t stream) {
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    using S = BwdDiagShape<N, P, CT>;
    static_assert(S::local_lds <= kMaxLds && S::terms_lds <= kMaxLds, "diagonal backward LDS budget");
    static bool attr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    if (!attr[dev]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_local_diag_kernel<T, N, P>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::local_lds) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_terms_diag_kernel<T, N, P>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::terms_lds) != hipSuccess)
            return -1;
        attr[dev] = true;
    }
    const int64_t units = bl.p.batch * bl.p.nheads, work = units * bl.p.nchunks;
    BwdParams p = bl.p;
    p.per_xcd = (units + 7) / 8;
    p.per_xcd_intra = (work + 7) / 8;
    int k = 0;
    if (units > 0) {
        // (seqlen 0: no chunks, so nothing to clear either; the scan still gives dinit = dfinal)
        if (work > 0 && !launch_k(bl, k, bwd_local_diag_kernel<T, N, P>, dim3((unsigned)(8 * p.per_xcd_intra)),
                                  dim3(kThreads), S::local_lds, stream, p))
            return -1;
        const int64_t scan_threads = 2 * units * N * P;
        if (!launch_k(bl, k, bwd_scan_diag_kernel<N, P>, dim3((unsigned)((scan_threads + kThreads - 1) / kThreads)),
                      dim3(kThreads), 0, stream, p))
            return -1;
        // (persistent: up to kBwdCUs workgroups, a multiple of 8, over the items)
        const int64_t wgs = std::min<int64_t>(kBwdCUs, (work + 7) / 8 * 8);
        if (work > 0 && !launch_k(bl, k, bwd_terms_diag_kernel<T, N, P>, dim3((unsigned)wgs), dim3(kBThreads),
                                  S::terms_lds, stream, p))
            return -1;
    }
    if (p.dD && !launch_k(bl, k, bwd_reduce_kernel, dim3((unsigned)bl.p.nheads),
                          dim3(kThreads), 0, stream, (const float*)p.dD_part, p.dD, bl.p.batch, bl.p.nheads,
                          (int64_t)bl.p.nchunks))
        return -1;
    return 0;
}

#define SSD_BWD_DIAG_SHAPES(X) X(16, 16) X(16, 32) X(16, 64) X(32, 16) X(32, 32) X(32, 64) X(64, 16) X(64, 32) X(64, 64)

#define SSD_BWD_SHAPES(X) \
    X(16, 16) X(16, 32) X(16, 64) X(32, 16) X(32, 32) X(32, 64) X(64, 16) X(64, 32) X(64, 64) X(128, 16) X(128, 32) X(128, 64)

}  // namespace

bool backward_shape_supported(int N, int P, int decay) {
#define SSD_BWD_MATCH(NN, PP) \
    if (N == NN && P == PP) return true;
    if (decay == 1) {
        SSD_BWD_DIAG_SHAPES(SSD_BWD_MATCH)
        return false;
    }
    SSD_BWD_SHAPES(SSD_BWD_MATCH)
#undef SSD_BWD_MATCH
    return false;
}

namespace {
// Workspace of the backward pass: checkpoints [B,H,nchunks,N,P] fp32 and per-(batch, head) dD sums
// (per (batch, head, chunk) for the diagonal decay); with the diagonal decay also the gradient
// slots [B,H,nchunks,N,P], e_last [B,H,nchunks,N] and the intra-chunk terms dx [B,T,H,P] and dB,
// dC, dcum [B,T,H,N], all fp32.
struct BwdLayout {
    size_t ckpt, part, gst, elw, dxi, dBi, dCi, dcumi, total;
};
BwdLayout bwd_layout(int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, int decay) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const int64_t nchunks = (seqlen + kBQ - 1) / kBQ;
    const size_t rows = (size_t)batch * (size_t)seqlen * (size_t)nheads;
    BwdLayout l{};
    size_t off = 0;
    l.ckpt = off; off = up(off + (size_t)(batch * nheads * nchunks) * (size_t)N * (size_t)P * 4);
    l.part = off; off = up(off + (size_t)(batch * nheads) * (size_t)(decay == 1 ? nchunks : 1) * 4);
    if (decay == 1) {
        l.gst = off; off = up(off + (size_t)(batch * nheads * nchunks) * (size_t)N * (size_t)P * 4);
        l.elw = off; off = up(off + (size_t)(batch * nheads * nchunks) * (size_t)N * 4);
        l.dxi = off; off = up(off + rows * P * 4);
        l.dBi = off; off = up(off + rows * N * 4);
        l.dCi = off; off = up(off + rows * N * 4);
        l.dcumi = off; off = up(off + rows * N * 4);
    }
    l.total = off;
    return l;
}
}  // namespace

size_t backward_workspace_bytes(int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, int decay) {
    return bwd_layout(batch, nheads, seqlen, N, P, decay).total;
}

void bind_backward_workspace(BwdParams& p, void* ws, int N, int P, int decay) {
    const BwdLayout l = bwd_layout(p.batch, p.nheads, p.seqlen, N, P, decay);
    char* w = static_cast<char*>(ws);
    auto at = [&](size_t off) { return w ? reinterpret_cast<float*>(w + off) : nullptr; };
    p.ckpt = at(l.ckpt);
    p.dD_part = at(l.part);
    p.gst = decay == 1 ? at(l.gst) : nullptr;
    p.elw = decay == 1 ? at(l.elw) : nullptr;
    p.dxi = decay == 1 ? at(l.dxi) : nullptr;
    p.dBi = decay == 1 ? at(l.dBi) : nullptr;
    p.dCi = decay == 1 ? at(l.dCi) : nullptr;
    p.dcumi = decay == 1 ? at(l.dcumi) : nullptr;
}

int launch_backward(const BackwardLaunch& bl, hipStream_t stream) {
    const int N = (int)bl.dstate, P = (int)bl.headdim;
    if (bl.decay == 1) {
#define SSD_BWD_DLAUNCH(NN, PP)                                                           \
    if (N == NN && P == PP)                                                               \
        return bl.dtype == 0 ? launch_backward_diag_t<float, NN, PP>(bl, stream)          \
                             : launch_backward_diag_t<__bf16, NN, PP>(bl, stream);
        SSD_BWD_DIAG_SHAPES(SSD_BWD_DLAUNCH)
#undef SSD_BWD_DLAUNCH
        return -2;
    }
#define SSD_BWD_LAUNCH(NN, PP)                                                             \
    if (N == NN && P == PP)                                                                \
        return bl.dtype == 0 ? launch_backward_t<float, NN, PP>(bl, stream)              \
                             : launch_backward_t<__bf16, NN, PP>(bl, stream);
    SSD_BWD_SHAPES(SSD_BWD_LAUNCH)
#undef SSD_BWD_LAUNCH
    return -2;
}

int backward_chunk() { return kBQ; }

DtBackwardLayout dt_backward_layout(int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, int elem_bytes,
                                    bool scale_input, int decay) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t rows = (size_t)batch * (size_t)seqlen * (size_t)nheads;
    const size_t K = decay == 1 ? (size_t)N : 1;
    DtBackwardLayout l;
    size_t off = 0;
    l.la = off; off = up(off + rows * K * 4);
    l.xs = off; if (scale_input) off = up(off + rows * P * elem_bytes);
    l.dxs = off; off = up(off + rows * P * elem_bytes);
    l.dla = off; off = up(off + rows * K * 4);
    l.ddt_rows = 0;  // (the caller's ddt holds them)
    l.rowA = off; off = up(off + rows * K * 4);
    l.rowD = off; off = up(off + rows * 4);
    l.inner = off; off += backward_workspace_bytes(batch, nheads, seqlen, N, P, decay);
    l.total = off;
    return l;
}

int launch_backward_dt(const BackwardLaunch& bl0, const DtBackwardArgs& a, hipStream_t stream) {
    // (a packed batch: its tokens, at most batch * seqlen, which the workspace rows are sized for)
    const int64_t bt = bl0.p.seq_off ? bl0.p.total : bl0.p.batch * bl0.p.seqlen;
    const int64_t H = bl0.p.nheads, rows = bt * H;
    const int P = (int)bl0.headdim;
    const int eb = bl0.dtype == 0 ? 4 : 2;
    const int K = bl0.decay == 1 ? (int)bl0.dstate : 1;
    const DtBackwardLayout l =
        dt_backward_layout(bl0.p.batch, H, bl0.p.seqlen, (int)bl0.dstate, P, eb, a.scale_input != 0, bl0.decay);
    char* ws = static_cast<char*>(a.workspace);
    float* la = reinterpret_cast<float*>(ws + l.la);
    void* xs = a.scale_input ? static_cast<void*>(ws + l.xs) : nullptr;
    void* dxs = ws + l.dxs;
    float* dla = reinterpret_cast<float*>(ws + l.dla);
    float* rowA = reinterpret_cast<float*>(ws + l.rowA);
    float* rowD = reinterpret_cast<float*>(ws + l.rowD);
    const unsigned grid = (unsigned)((rows + kThreads - 1) / kThreads);
    if (rows > 0) {
        if (bl0.dtype == 0)
            hipLaunchKernelGGL(disc_rows_kernel<float>, dim3(grid), dim3(kThreads), 0, stream, a.dt, a.dt_bias, a.A_log,
                               static_cast<const float*>(a.x), la, static_cast<float*>(xs), rows, H, P, K);
        else
            hipLaunchKernelGGL(disc_rows_kernel<__bf16>, dim3(grid), dim3(kThreads), 0, stream, a.dt, a.dt_bias,
                               a.A_log, static_cast<const __bf16*>(a.x), la, static_cast<__bf16*>(xs), rows, H, P, K);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    // the backward pass on (x_in, log a) with no skip term; dx_in and dlog a into the workspace
    BackwardLaunch bl = bl0;
    bl.p.x = xs ? xs : a.x;
    bl.p.log_a = la;
    bl.p.D = nullptr;
    bl.p.dx = dxs;
    bl.p.dlog_a = dla;
    bl.p.dD = nullptr;
    bind_backward_workspace(bl.p, ws + l.inner, (int)bl0.dstate, P, bl0.decay);
    const int rc = launch_backward(bl, stream);
    if (rc != 0) return rc;
    if (rows > 0) {
        if (bl0.dtype == 0)
            hipLaunchKernelGGL(disc_grad_rows_kernel<float>, dim3(grid), dim3(kThreads), 0, stream, a.dt, a.dt_bias,
                               a.A_log, a.D, static_cast<const float*>(a.x), static_cast<const float*>(a.dy),
                               static_cast<const float*>(dxs), la, dla, a.scale_input, static_cast<float*>(a.dx), a.ddt,
                               rowA, rowD, rows, H, P, K);
        else
            hipLaunchKernelGGL(disc_grad_rows_kernel<__bf16>, dim3(grid), dim3(kThreads), 0, stream, a.dt, a.dt_bias,
                               a.A_log, a.D, static_cast<const __bf16*>(a.x), static_cast<const __bf16*>(a.dy),
                               static_cast<const __bf16*>(dxs), la, dla, a.scale_input, static_cast<__bf16*>(a.dx),
                               a.ddt, rowA, rowD, rows, H, P, K);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (a.ddt_bias) hipLaunchKernelGGL(head_sum_kernel, dim3((unsigned)H), dim3(kThreads), 0, stream, a.ddt, a.ddt_bias, bt, H);
    if (a.dA_log)
        hipLaunchKernelGGL(head_sum_kernel, dim3((unsigned)(H * K)), dim3(kThreads), 0, stream, rowA, a.dA_log, bt, H * K);
    if (a.dD) hipLaunchKernelGGL(head_sum_kernel, dim3((unsigned)H), dim3(kThreads), 0, stream, rowD, a.dD, bt, H);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace ssd
