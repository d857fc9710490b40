// HIP kernels of the chunked SSD forward and the decode step, for gfx950 (MI355X).
//
// Forward = two launches per call:
//   scores_kernel  S = C B^T for every (batch, group, chunk): the query-key products of the
//                  attention form (llms.blog "The SSD Theoretical Equivalence": Q = C, K = B),
//                  computed once per group and shared by all its heads.  Only the causal
//                  16x16 tiles (s <= t) are formed, stored fp32 in MFMA accumulator order.
//   walk_kernel    one workgroup per (batch, head) walks the chunks in order, keeping the
//                  N x P fp32 state in registers (aiwiki "State Space Duality", "Two
//                  algorithms for one operator"; llms.blog "The Chunk-Wise SSD Algorithm"):
//                    y_chunk = (S o L) X  +  exp(cum_t) C_t H_{k-1}  +  D x
//                    H_k     = exp(cum_last) H_{k-1} + (exp(cum_last - cum_s) B_s)^T X
//                  with L_ts = exp(cum_t - cum_s) for s <= t (selected before the exp) and
//                  cum the running sum of log a inside the chunk.  Each workgroup reads its
//                  x once and writes y once; the state never leaves the chip.
//
// MFMA tiling (16x16 tiles, 4 waves of 64 lanes): the accumulator of a 16x16 MFMA holds,
// in lane l, rows 4*(l/16)+i (i = 0..3) of column l%16.  Products whose operand comes out
// of an accumulator (the masked scores, the state) use it in place by giving each lane
// group the K indices its accumulator rows hold; the partner operand is read from LDS in
// the same K order.  Everything a lane reads or writes along a row is 8 or 16 bytes wide.

#include <algorithm>
#include <type_traits>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

template <typename T> __device__ __forceinline__ T vec_elem(uint4 u, int j);
template <> __device__ __forceinline__ __bf16 vec_elem<__bf16>(uint4 u, int j) { return as_bf16x8(u)[j]; }
template <> __device__ __forceinline__ float vec_elem<float>(uint4 u, int j) { return as_f32x4(u)[j]; }

// Four consecutive elements into LDS (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ void lds_store4(__bf16* p, __bf16 a, __bf16 b, __bf16 c, __bf16 d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<bf16x4*>(p) = bf16x4{a, b, c, d};
}
__device__ __forceinline__ void lds_store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// acc += A_blk * B_blk over one K block; a and b are a lane's 16 bytes of each operand.
__device__ __forceinline__ f32x4 mma_block(f32x4 acc, uint4 a, uint4 b, __bf16) {
    return mfma_bf16(as_bf16x8(a), as_bf16x8(b), acc);
}
__device__ __forceinline__ f32x4 mma_block(f32x4 acc, uint4 a, uint4 b, float) {
    const f32x4 av = as_f32x4(a), bv = as_f32x4(b);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma_f32(av[i], bv[i], acc);
    return acc;
}

// exp of a non-positive log-decay difference.  fp32 inputs keep the running sums in fp64
// and use the accurate expf; bf16 inputs use the hardware exp2-based __expf.
__device__ __forceinline__ float decay_exp(double d) { return expf((float)d); }
__device__ __forceinline__ float decay_exp(float d) { return __expf(d); }

__host__ __device__ constexpr int tile_index(int tb, int sb) { return tb * (tb + 1) / 2 + sb; }
// score tiles of a block row that the walk reads ahead of the carried-state products: four for
// states of up to 4096 elements, none above (where the registers are needed for the state)
template <int N, int P> constexpr int pre_tiles() { return N * P <= 4096 ? 4 : 0; }

// ---------------------------------------------------------------------------------------
// scores_kernel: one workgroup per (batch, group, chunk); wave w forms causal tiles
// w, w+4, ...  Tile (tb, sb) holds S^T[s][t] = C_t . B_s for s in block sb, t in block tb,
// lane l storing its 4 accumulator values at offset 4*l.
template <typename T, int N>
__global__ void __launch_bounds__(kThreads) scores_kernel(ScoresParams prm) {
    using TR = Traits<T>;
    constexpr int KB = TR::kKBlock;
    const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int l16 = lane % 16, lg = lane / 16;
    const int64_t blk = blockIdx.x;
    const int c = (int)(blk % prm.nchunks);
    const int64_t bg = blk / prm.nchunks;
    const int64_t b = bg / prm.ngroups;
    const int64_t g = bg % prm.ngroups;
    const int Q = prm.chunk, nt = Q / 16, ntiles = nt * (nt + 1) / 2;
    const int64_t t0 = (int64_t)c * Q;
    const SeqSpan sq = seq_span(prm.seq_off, b, prm.seqlen, prm.total);
    if (t0 >= sq.len) return;  // (a packed sequence shorter than seqlen: no such chunk)
    const int len = (int)min((int64_t)Q, sq.len - t0);
    const T* Bm = static_cast<const T*>(prm.Bm);
    const T* Cm = static_cast<const T*>(prm.Cm);
    float* out = prm.scores + blk * (int64_t)ntiles * 256;
    const uint4 zero = {0u, 0u, 0u, 0u};

    int idx = 0;
    for (int tb = 0; tb < nt; ++tb) {
        for (int sb = 0; sb <= tb; ++sb, ++idx) {
            if (idx % kWaves != wave) continue;
            const int s = 16 * sb + l16, t = 16 * tb + l16;
            const T* brow = Bm + ((sq.row0 + t0 + s) * prm.ngroups + g) * N;
            const T* crow = Cm + ((sq.row0 + t0 + t) * prm.ngroups + g) * N;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < N / KB; ++kb) {
                const int k0 = kb * KB + (KB / 4) * lg;
                const uint4 av = s < len ? ld16(brow + k0) : zero;
                const uint4 bv = t < len ? ld16(crow + k0) : zero;
                acc = mma_block(acc, av, bv, T());
            }
            *reinterpret_cast<f32x4*>(out + idx * 256 + lane * 4) = acc;
        }
    }
}

// ---------------------------------------------------------------------------------------
// walk_kernel: one workgroup per (batch, head); see the file header.
//
// LDS:  Xt [P][QP]  x of the chunk, transposed (tokens contiguous)
//       Bt [N][QP]  (exp(cum_last - cum_s) * B_s) of the chunk, transposed
//       Ht [P][NP]  the state entering the chunk, transposed (state dims contiguous), in T
//       cum[256]    running log-decay sums of the chunk
// Registers: the fp32 state, tiles (nb, pb) dealt to the 4 waves round-robin; the output
// accumulators of one 16-token block at a time (blocks dealt to waves round-robin).
template <typename T, int N, int P>
__global__ void __launch_bounds__(kThreads) walk_kernel(WalkParams prm) {
    using TR = Traits<T>;
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    constexpr int KB = TR::kKBlock;
    constexpr int VE = TR::kVec;
    constexpr int PB = P / 16;
    constexpr int NB = N / 16;
    constexpr int NTILE = NB * PB;
    constexpr int TPW = (NTILE + kWaves - 1) / kWaves;
    constexpr int NP = N + TR::kPad;
    constexpr int kPre = pre_tiles<N, P>();

    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, prm.batch * H);
    if (unit < 0) return;
    const int64_t b = unit / H;
    const int64_t h = unit % H;
    const int64_t g = h / (H / G);
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);

    const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, lg = lane / 16;
    const int koff = (KB / 4) * lg;  // this lane group's first K index inside a K block
    const int Q = prm.chunk;
    const int nch = (int)((sq.len + Q - 1) / Q);
    const int QK = (Q + KB - 1) / KB * KB;
    const int QP = QK + TR::kPad;
    const int nt = Q / 16;
    const int ntiles = nt * (nt + 1) / 2;

    extern __shared__ __align__(16) unsigned char smem[];
    T* Xt = reinterpret_cast<T*>(smem);
    T* Bt = Xt + P * QP;
    T* Ht = Bt + N * QP;
    CT* cum = reinterpret_cast<CT*>(Ht + P * NP);
    CT* scan_tmp = cum + 256;

    const T* xg = static_cast<const T*>(prm.x);
    const T* Bg = static_cast<const T*>(prm.Bm);
    const T* Cg = static_cast<const T*>(prm.Cm);
    T* yg = static_cast<T*>(prm.y);
    const uint4 zero = {0u, 0u, 0u, 0u};

    // ---- state registers, from init_state or zero
    f32x4 hs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        hs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wave + kWaves * j;
        if (tile < NTILE && prm.init) {
            const int nb = tile / PB, pb = tile % PB;
            const float* src = prm.init + (unit * N + 16 * nb + 4 * lg) * P + 16 * pb + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) hs[j][i] = src[i * P];
        }
    }
    auto write_state_lds = [&]() {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                lds_store4(Ht + (16 * pb + l16) * NP + 16 * nb + 4 * lg, (T)hs[j][0], (T)hs[j][1],
                           (T)hs[j][2], (T)hs[j][3]);
            }
        }
    };
    write_state_lds();

    const float dskip = prm.D ? prm.D[h] : 0.f;
    const float* scores_bg = prm.scores + (b * G + g) * (int64_t)prm.nchunks * ntiles * 256;
    // log a of token tid of chunk cc (0 past the sequence end), loaded a chunk ahead of its use
    auto load_la = [&](int cc) -> CT {
        const int64_t tt = (int64_t)cc * Q + tid;
        return (tid < Q && tt < sq.len) ? (CT)prm.log_a[(sq.row0 + tt) * H + h] : (CT)0;
    };
    CT la_next = load_la(0);

    for (int c = 0; c < nch; ++c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);

        // ---- 1. running sum of log a inside the chunk (tokens past the end add 0)
        CT v = block_inclusive_scan(la_next, scan_tmp);
        if (tid < Q) cum[tid] = v;
        la_next = load_la(c + 1);
        __syncthreads();
        const CT cum_last = cum[Q - 1];

        // ---- 2. stage x^T and (w o B)^T; rows past the chunk's end are zero
        for (int item = tid; item < (QK / 4) * (P / VE); item += kThreads) {
            const int rg = item / (P / VE), cc = item % (P / VE);
            uint4 u[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 4 * rg + k;
                u[k] = r < len ? ld16(xg + ((sq.row0 + t0 + r) * H + h) * P + cc * VE) : zero;
            }
#pragma unroll
            for (int j = 0; j < VE; ++j)
                lds_store4(Xt + (cc * VE + j) * QP + 4 * rg, vec_elem<T>(u[0], j), vec_elem<T>(u[1], j),
                           vec_elem<T>(u[2], j), vec_elem<T>(u[3], j));
        }
        for (int item = tid; item < (QK / 4) * (N / VE); item += kThreads) {
            const int rg = item / (N / VE), cc = item % (N / VE);
            uint4 u[4];
            float w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 4 * rg + k;
                const bool ok = r < len;
                u[k] = ok ? ld16(Bg + ((sq.row0 + t0 + r) * G + g) * N + cc * VE) : zero;
                w[k] = ok ? decay_exp(cum_last - cum[r]) : 0.f;
            }
#pragma unroll
            for (int j = 0; j < VE; ++j)
                lds_store4(Bt + (cc * VE + j) * QP + 4 * rg,
                           from_f32<T>(w[0] * to_f32(vec_elem<T>(u[0], j))),
                           from_f32<T>(w[1] * to_f32(vec_elem<T>(u[1], j))),
                           from_f32<T>(w[2] * to_f32(vec_elem<T>(u[2], j))),
                           from_f32<T>(w[3] * to_f32(vec_elem<T>(u[3], j))));
        }
        __syncthreads();

        // ---- 3. outputs: y^T[p][t] for 16-token blocks tb = wave, wave+4, ...
        const float* scores_c = scores_bg + (int64_t)c * ntiles * 256;
        for (int tb = wave; tb < nt; tb += kWaves) {
            const int tl = 16 * tb + l16;  // this lane's token inside the chunk
            const bool tvalid = tl < len;
            const int64_t trow = sq.row0 + t0 + tl;
            f32x4 acc[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
            // the first kPre score tiles of this block row, read now so that their latency
            // overlaps the carried-state products (the rest are read where they are used)
            auto load_tile = [&](int sb) -> f32x4 {
                return as_f32x4(ld16(scores_c + tile_index(tb, sb) * 256 + lane * 4));
            };
            f32x4 pre[kPre > 0 ? kPre : 1];
#pragma unroll
            for (int i = 0; i < kPre; ++i) pre[i] = i <= tb ? load_tile(i) : f32x4{0.f, 0.f, 0.f, 0.f};

            // carried state: C_t . H_{k-1}, then the decay from the chunk start, exp(cum_t)
            const T* crow = Cg + (trow * G + g) * N;
#pragma unroll
            for (int kb = 0; kb < N / KB; ++kb) {
                const uint4 cv = tvalid ? ld16(crow + kb * KB + koff) : zero;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
                    acc[pb] = mma_block(acc[pb], ld16(Ht + (16 * pb + l16) * NP + kb * KB + koff), cv, T());
            }
            const CT cum_t = cum[tl];
            const float ec = decay_exp(cum_t);
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[pb] *= ec;

            // within the chunk: (S o L) X, mask selected before the exp; the first kPre tiles come
            // from the registers read above (sb is uniform over the wave: a scalar branch)
            auto masked_tile = [&](int sb) -> f32x4 {
                f32x4 s4;
                if constexpr (kPre > 0) {
                    if (sb < kPre) {
                        s4 = pre[0];
#pragma unroll
                        for (int i = 1; i < kPre; ++i) s4 = sb == i ? pre[i] : s4;
                    } else {
                        s4 = load_tile(sb);
                    }
                } else {
                    s4 = load_tile(sb);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 16 * sb + 4 * lg + i;
                    const bool causal = s <= tl;
                    const CT d = causal ? (CT)(cum_t - cum[s]) : (CT)0;
                    s4[i] = causal ? s4[i] * decay_exp(d) : 0.f;
                }
                return s4;
            };
            if constexpr (std::is_same<T, __bf16>::value) {
                for (int k = 0; 2 * k <= tb; ++k) {
                    const f32x4 m0 = masked_tile(2 * k);
                    const f32x4 m1 = (2 * k + 1 <= tb) ? masked_tile(2 * k + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
                    const bf16x8 bop = {(__bf16)m0[0], (__bf16)m0[1], (__bf16)m0[2], (__bf16)m0[3],
                                        (__bf16)m1[0], (__bf16)m1[1], (__bf16)m1[2], (__bf16)m1[3]};
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const T* xr = Xt + (16 * pb + l16) * QP + 32 * k + 4 * lg;
                        const uint2 lo = ld8(xr), hi = ld8(xr + 16);
                        const uint4 a = {lo.x, lo.y, hi.x, hi.y};
                        acc[pb] = mfma_bf16(as_bf16x8(a), bop, acc[pb]);
                    }
                }
            } else {
                for (int sb = 0; sb <= tb; ++sb) {
                    const f32x4 m = masked_tile(sb);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const f32x4 xa = as_f32x4(ld16(Xt + (16 * pb + l16) * QP + 16 * sb + 4 * lg));
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[pb] = mfma_f32(xa[i], m[i], acc[pb]);
                    }
                }
            }

            // skip term and store
            if (prm.D) {
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[pb][i] += dskip * to_f32(Xt[(16 * pb + 4 * lg + i) * QP + tl]);
            }
            if (tvalid) {
                T* yr = yg + (trow * H + h) * P + 4 * lg;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
                    store4(yr + 16 * pb, acc[pb][0], acc[pb][1], acc[pb][2], acc[pb][3]);
            }
        }

        // ---- 4. state: H_k = exp(cum_last) H_{k-1} + (w o B)^T X
        const float el = decay_exp(cum_last);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                f32x4 a = hs[j] * el;
                const T* br = Bt + (16 * nb + l16) * QP + koff;
                const T* xr = Xt + (16 * pb + l16) * QP + koff;
                for (int kb = 0; kb < QK / KB; ++kb) a = mma_block(a, ld16(br + kb * KB), ld16(xr + kb * KB), T());
                hs[j] = a;
            }
        }
        __syncthreads();
        write_state_lds();
    }

    if (prm.final_state) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                float* dst = prm.final_state + (unit * N + 16 * nb + 4 * lg) * P + 16 * pb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * P] = hs[j][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Decode step (llms.blog "The Duality of Inference and Training in Linear Time-Invariant
// SSMs": the recurrent mode, one token at a time): h <- a h + B_t x_t^T, y_t = C_t^T h + D x_t.
// One 256-thread workgroup per (batch, head).  Thread (r, q) owns columns 4q .. 4q + 3 of the
// state rows r RPT .. r RPT + RPT - 1; it issues every load of its rows (16 bytes each, with
// the rows' B, C and decays) before its first FMA, so a workgroup has the whole 32 KiB state of
// its head in flight at once, then writes its rows back and reduces its part of the readout
// over the row groups (wave shuffles, then one LDS exchange between the four waves).
template <typename T, int RPT>
__device__ __forceinline__ void load_rows(const T* src, float (&v)[RPT]) {
    if constexpr ((RPT * sizeof(T)) % 16 == 0) {
        constexpr int E = 16 / sizeof(T), L = RPT / E;
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const uint4 w = ld16(src + E * l);
            if constexpr (sizeof(T) == 4) {
                const f32x4 f = as_f32x4(w);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * l + e] = f[e];
            } else {
                const bf16x8 f = as_bf16x8(w);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[8 * l + e] = (float)f[e];
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < RPT; ++k) v[k] = to_f32(src[k]);
    }
}

template <typename T, int RPT>
__global__ void __launch_bounds__(kThreads) step_kernel(StepParams prm) {
    const int64_t unit = blockIdx.x;
    const int64_t H = prm.nheads, G = prm.ngroups;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const int P = prm.headdim, N = prm.dstate;
    const int QP = P / 4;                      // column quads per row
    const int q = threadIdx.x % QP, r = threadIdx.x / QP;
    const int n0 = r * RPT;                    // first row of this thread
    const bool active = n0 < N;                // (more row groups than rows for small N)
    const int nrow = active ? n0 : 0;
    const T* __restrict__ xt = static_cast<const T*>(prm.x_t) + unit * P + 4 * q;
    const T* __restrict__ Bt = static_cast<const T*>(prm.B_t) + (b * G + g) * N + nrow;
    const T* __restrict__ Ct = static_cast<const T*>(prm.C_t) + (b * G + g) * N + nrow;
    float* __restrict__ st = prm.state + unit * N * P + (int64_t)nrow * P + 4 * q;

    // every load first: the state rows, x, B, C and the decays of this thread's rows
    f32x4 s[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) s[k] = *reinterpret_cast<const f32x4*>(st + k * P);
    float xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = to_f32(xt[i]);
    const float d = prm.D ? prm.D[h] : 0.f;  // (loaded with the rest, not after the reduction)
    float bv[RPT], cv[RPT];
    load_rows<T, RPT>(Bt, bv);
    load_rows<T, RPT>(Ct, cv);
    // with the discretisation front-end: Delta = softplus(dt + bias), log a = -Delta exp(A_log)
    // (per head, or per (head, n)), and the input term scaled by Delta
    const bool disc = prm.dt_t != nullptr;
    const float delta = disc ? softplusf(prm.dt_t[unit] + (prm.dt_bias ? prm.dt_bias[h] : 0.f)) : 0.f;
    float av[RPT];  // the decay factor a of each row
    if (prm.diag) {
        load_rows<float, RPT>(disc ? prm.A_log + h * N + nrow : prm.log_a_t + unit * N + nrow, av);
#pragma unroll
        for (int k = 0; k < RPT; ++k) av[k] = expf(disc ? -delta * expf(av[k]) : av[k]);
    } else {
        const float a = expf(disc ? -delta * expf(prm.A_log[h]) : prm.log_a_t[unit]);
#pragma unroll
        for (int k = 0; k < RPT; ++k) av[k] = a;
    }
    const float sc = disc && prm.scale_input ? delta : 1.f;
    float xin[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xin[i] = sc * xv[i];

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[k][i] = av[k] * s[k][i] + bv[k] * xin[i];
            acc[i] += cv[k] * s[k][i];
        }
    }
    if (active)  // (an active thread's rows all lie below N: N is a multiple of RPT)
#pragma unroll
        for (int k = 0; k < RPT; ++k) *reinterpret_cast<f32x4*>(st + k * P) = s[k];
    if (!active) acc = f32x4{0.f, 0.f, 0.f, 0.f};
    // partial readouts of the row groups of one column quad: first inside the wave ...
#pragma unroll
    for (int off = QP; off < kWave; off <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off, kWave);
    // ... then between the waves
    __shared__ f32x4 red[kWaves][kWave];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    if (lane < QP) red[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x < QP) {
        f32x4 y = red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) y += red[w][threadIdx.x];
        store4(static_cast<T*>(prm.y_t) + unit * P + 4 * q, y[0] + d * xv[0], y[1] + d * xv[1], y[2] + d * xv[2],
               y[3] + d * xv[3]);
    }
}

// final_state = init_state (or zeros) for an empty sequence.
__global__ void __launch_bounds__(kThreads) copy_state_kernel(const float* src, float* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// Discretisation front-end for the generic paths: per (b, t, h), Delta = softplus(dt + bias),
// log a = -Delta exp(A_log) written to la ([B,T,H] with K = 1, or [B,T,H,N] with K = N and
// A_log [H,N]), and with xs non-null the scaled input Delta x written to xs.  In double, so
// that the fp32 path's log a carries only its final rounding.
template <typename T>
__global__ void __launch_bounds__(kThreads) discretize_kernel(const float* dt, const float* dt_bias,
                                                              const float* A_log, const T* x, float* la, T* xs,
                                                              int64_t tokens, int64_t nheads, int K, int P) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < tokens * K; i += stride) {
        const int64_t th = i / K;  // (b, t, h) row
        const int64_t h = th % nheads;
        const int k = (int)(i % K);
        const double delta = softplus((double)dt[th] + (dt_bias ? (double)dt_bias[h] : 0.0));
        la[i] = (float)(-delta * exp((double)A_log[h * K + k]));
    }
    if (!xs) return;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < tokens * P; i += stride) {
        const int64_t th = i / P;
        const int64_t h = th % nheads;
        const double delta = softplus((double)dt[th] + (dt_bias ? (double)dt_bias[h] : 0.0));
        xs[i] = from_f32<T>((float)(delta * (double)to_f32(x[i])));
    }
}

// y += D[h] x over [B,T,H,P]: the skip term on the raw input, after a walk that ran on the
// scaled input without one.
template <typename T>
__global__ void __launch_bounds__(kThreads) skip_kernel(const T* x, const float* D, T* y, int64_t n, int64_t nheads,
                                                        int P) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const int64_t h = (i / P) % nheads;
        y[i] = from_f32<T>(to_f32(y[i]) + D[h] * to_f32(x[i]));
    }
}

template <typename T>
int launch_forward_discretized_t(const ForwardLaunch& fl, hipStream_t stream) {
    const int K = fl.decay == 1 ? (int)fl.dstate : 1;
    const int P = (int)fl.headdim;
    const size_t own = generic_workspace_bytes(fl.dtype, fl.decay, fl.batch, fl.nheads, fl.ngroups, fl.seqlen,
                                               (int)fl.dstate, P, fl.chunk);
    const DtGenericLayout lay = dt_generic_layout(own, fl.batch, fl.seqlen, fl.nheads, K, P, (int)sizeof(T),
                                                  fl.scale_input != 0);
    char* ws = reinterpret_cast<char*>(fl.scores);
    float* la = reinterpret_cast<float*>(ws + lay.la);
    T* xs = fl.scale_input ? reinterpret_cast<T*>(ws + lay.xs) : nullptr;
    // (a packed batch: its tokens, which the caller's contract keeps within batch * seqlen, the
    // size of the workspace rows)
    const int64_t tokens = (fl.seq_off ? fl.total : fl.batch * fl.seqlen) * fl.nheads;
    const int64_t work = tokens * (K > P ? K : P);
    const unsigned grid = (unsigned)std::min<int64_t>((work + kThreads - 1) / kThreads, 8192);
    int k = fl.first_launch;
    if (!launch_k(fl, k, discretize_kernel<T>, dim3(grid), dim3(kThreads), 0, stream, fl.dt, fl.dt_bias, fl.A_log,
                  static_cast<const T*>(fl.x), la, xs, tokens, fl.nheads, K, P))
        return -1;
    // the walk on log a and (with the input scale) the scaled input; then the skip term
    ForwardLaunch g = fl;
    g.dt = g.dt_bias = g.A_log = nullptr;
    g.scale_input = 0;
    g.log_a = la;
    g.first_launch = k;
    if (xs) {
        g.x = xs;
        g.D = nullptr;
    }
    const int rc = launch_forward(g, stream);
    if (rc != 0) return rc;
    if (xs && fl.D) {
        k = *fl.n_launches;
        const int64_t n = tokens * P;
        const unsigned sgrid = (unsigned)std::min<int64_t>((n + kThreads - 1) / kThreads, 8192);
        if (!launch_k(fl, k, skip_kernel<T>, dim3(sgrid), dim3(kThreads), 0, stream, static_cast<const T*>(fl.x), fl.D,
                      static_cast<T*>(fl.y), n, fl.nheads, P))
            return -1;
    }
    return 0;
}

// ---------------------------------------------------------------------------------------
template <typename T> constexpr int kBytes = sizeof(T);

template <typename T, int N, int P>
size_t walk_lds_bytes_t(int chunk) {
    const int KB = Traits<T>::kKBlock;
    const int QK = (chunk + KB - 1) / KB * KB;
    const int QP = QK + Traits<T>::kPad;
    const int NP = N + Traits<T>::kPad;
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    return (size_t)(P * QP + N * QP + P * NP) * sizeof(T) + (256 + kWaves) * sizeof(CT);
}

template <typename T, int N, int P>
int launch_forward_t(const ForwardLaunch& fl, hipStream_t stream) {
    const int Q = fl.chunk;
    const int nt = Q / 16;
    const int ntiles = nt * (nt + 1) / 2;
    ScoresParams sp{fl.Bm, fl.Cm, fl.scores, fl.seqlen, fl.ngroups, Q, fl.nchunks, fl.seq_off, fl.total};
    const int64_t nscore = fl.batch * fl.ngroups * fl.nchunks;
    (void)ntiles;
    int k = fl.first_launch;
    if (!launch_k(fl, k, scores_kernel<T, N>, dim3((unsigned)nscore), dim3(kThreads), 0, stream, sp)) return -1;

    const int64_t units = fl.batch * fl.nheads;
    const int64_t per_xcd = (units + 7) / 8;
    WalkParams wp{fl.x, fl.log_a, fl.Bm, fl.Cm, fl.D, fl.scores, fl.init, fl.y, fl.final_state,
                  fl.batch, fl.seqlen, fl.nheads, fl.ngroups, Q, fl.nchunks, per_xcd};
    wp.seq_off = fl.seq_off;
    wp.total = fl.total;
    const size_t lds = walk_lds_bytes_t<T, N, P>(Q);
    // Allow the full 160 KiB of LDS, once per device.
    static bool attr_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    if (!attr_set[dev]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&walk_kernel<T, N, P>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) != hipSuccess)
            return -1;
        attr_set[dev] = true;
    }
    return launch_k(fl, k, walk_kernel<T, N, P>, dim3((unsigned)(8 * per_xcd)), dim3(kThreads), lds, stream, wp)
               ? 0
               : -1;
}

// The (element type, N, P) instantiations the library ships.
#define SSD_FOR_EACH_SHAPE(X)                                                                       \
    X(__bf16, 32, 16) X(__bf16, 32, 32) X(__bf16, 32, 64) X(__bf16, 32, 128)                        \
    X(__bf16, 64, 16) X(__bf16, 64, 32) X(__bf16, 64, 64) X(__bf16, 64, 128)                        \
    X(__bf16, 128, 16) X(__bf16, 128, 32) X(__bf16, 128, 64) X(__bf16, 128, 128)                    \
    X(__bf16, 256, 16) X(__bf16, 256, 32) X(__bf16, 256, 64)                                        \
    X(float, 16, 16) X(float, 16, 32) X(float, 16, 64) X(float, 16, 128)                            \
    X(float, 32, 16) X(float, 32, 32) X(float, 32, 64) X(float, 32, 128)                            \
    X(float, 64, 16) X(float, 64, 32) X(float, 64, 64) X(float, 64, 128)                            \
    X(float, 128, 16) X(float, 128, 32) X(float, 128, 64) X(float, 128, 128)                        \
    X(float, 256, 16) X(float, 256, 32) X(float, 256, 64)

}  // namespace

bool shape_supported(int dtype, int N, int P) {
#define SSD_MATCH(TT, NN, PP) \
    if ((std::is_same<TT, float>::value ? 0 : 1) == dtype && N == NN && P == PP) return true;
    SSD_FOR_EACH_SHAPE(SSD_MATCH)
#undef SSD_MATCH
    return false;
}

size_t walk_lds_bytes(int dtype, int N, int P, int chunk) {
#define SSD_LDS(TT, NN, PP) \
    if ((std::is_same<TT, float>::value ? 0 : 1) == dtype && N == NN && P == PP) return walk_lds_bytes_t<TT, NN, PP>(chunk);
    SSD_FOR_EACH_SHAPE(SSD_LDS)
#undef SSD_LDS
    return 0;
}

size_t scores_bytes(int64_t batch, int64_t ngroups, int64_t nchunks, int chunk) {
    const int64_t nt = chunk / 16;
    return (size_t)(batch * ngroups * nchunks) * (size_t)(nt * (nt + 1) / 2) * 256 * sizeof(float);
}

size_t generic_workspace_bytes(int dtype, int decay, int64_t batch, int64_t nheads, int64_t ngroups, int64_t seqlen,
                               int N, int P, int chunk) {
    (void)dtype, (void)nheads, (void)N, (void)P;
    if (decay == 1) return 0;  // the unpipelined diagonal walk keeps everything on chip
    return scores_bytes(batch, ngroups, (seqlen + chunk - 1) / chunk, chunk);
}

int launch_forward(const ForwardLaunch& fl, hipStream_t stream) {
    if (fl.seqlen == 0) {
        if (fl.final_state) {
            const int64_t n = fl.batch * fl.nheads * fl.dstate * fl.headdim;
            if (n > 0) {
                int k = 0;
                if (!launch_k(fl, k, copy_state_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                              dim3(kThreads), 0, stream, fl.init, fl.final_state, n))
                    return -1;
            }
        }
        return 0;
    }
    if (fl.dt && !discretization_fused(fl.dtype, fl.decay, (int)fl.dstate, (int)fl.headdim, fl.chunk, fl.nheads,
                                       fl.ngroups))
        return fl.dtype == 0 ? launch_forward_discretized_t<float>(fl, stream)
                             : launch_forward_discretized_t<__bf16>(fl, stream);
    if (fl.decay == 1) return launch_forward_diag(fl, stream);
    if (fast_path_applies(fl.dtype, fl.decay, (int)fl.dstate, (int)fl.headdim, fl.chunk, fl.nheads, fl.ngroups))
        return launch_forward_fast(fl, stream);
#define SSD_LAUNCH(TT, NN, PP) \
    if ((std::is_same<TT, float>::value ? 0 : 1) == fl.dtype && fl.dstate == NN && fl.headdim == PP) \
        return launch_forward_t<TT, NN, PP>(fl, stream);
    SSD_FOR_EACH_SHAPE(SSD_LAUNCH)
#undef SSD_LAUNCH
    return -2;
}

template <typename T>
bool launch_step_t(const StepParams& sp, int64_t units, hipStream_t stream) {
    // rows per thread: the state's N rows over the 256 / (P / 4) row groups of a workgroup
    const int groups = kThreads / (sp.headdim / 4);
    const int rpt = (sp.dstate + groups - 1) / groups;
    const dim3 grid((unsigned)units), block(kThreads);
    switch (rpt) {
        case 1: hipLaunchKernelGGL((step_kernel<T, 1>), grid, block, 0, stream, sp); break;
        case 2: hipLaunchKernelGGL((step_kernel<T, 2>), grid, block, 0, stream, sp); break;
        case 4: hipLaunchKernelGGL((step_kernel<T, 4>), grid, block, 0, stream, sp); break;
        case 8: hipLaunchKernelGGL((step_kernel<T, 8>), grid, block, 0, stream, sp); break;
        case 16: hipLaunchKernelGGL((step_kernel<T, 16>), grid, block, 0, stream, sp); break;
        case 32: hipLaunchKernelGGL((step_kernel<T, 32>), grid, block, 0, stream, sp); break;
        default: return false;
    }
    return true;
}

int launch_step(const StepParams& sp, int dtype, int64_t units, hipStream_t stream) {
    if (units == 0) return 0;
    // (the supported shapes: P in {16, 32, 64, 128}, N in {16, ..., 256}, so 1 <= rows per thread <= 32)
    const bool ok = dtype == 0 ? launch_step_t<float>(sp, units, stream) : launch_step_t<__bf16>(sp, units, stream);
    if (!ok) return -2;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace ssd
