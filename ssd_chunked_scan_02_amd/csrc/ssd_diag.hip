// Chunked SSD forward with a diagonal transition: one decay per state dimension n,
// a_t = diag(exp(log_a[b,t,h,:])) ("On Structured State-Space Duality", ICML 2026 poster,
// abstract item (i); recurrence as in llms.blog "State Space Models and Mamba",
// "Continuous-to-Discrete Discretization").  Same chunk decomposition as the scalar case
// (aiwiki "State Space Duality", "Two algorithms for one operator"), with the decay inside the
// sum over n:
//   y_t   = sum_{s<=t in chunk} M_ts x_s + sum_n C_tn exp(cum_tn) H_{k-1}[n,:] + D x_t,
//   M_ts  = sum_n C_tn B_sn exp(cum_tn - cum_sn),
//   H_k[n,:] = exp(cum_last,n) H_{k-1}[n,:] + sum_s B_sn exp(cum_last,n - cum_sn) x_s,
// cum the running sum of log a inside the chunk, per n.
//
// Every exponential is of a non-positive number.  For a 16-token output block tb (first token
// a) and an earlier 16-token block sb (last token e), the mask of the score tile factors per n
// as exp(cum_t - cum_a) * exp(cum_a - cum_e) * exp(cum_e - cum_s), so the tile is one MFMA
// contraction over n of (C o f) diag(beta) and (B o u).  Diagonal tiles take the exact
// exponential per (t, s, n): within one block a single step's decay can exceed the fp32 range
// of any split into two factors.
//
// One workgroup (4 waves) per (batch, head) walks the chunks with the fp32 state in registers.

#include <type_traits>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

template <typename T> __device__ __forceinline__ T vec_elem(uint4 u, int j);
template <> __device__ __forceinline__ __bf16 vec_elem<__bf16>(uint4 u, int j) { return as_bf16x8(u)[j]; }
template <> __device__ __forceinline__ float vec_elem<float>(uint4 u, int j) { return as_f32x4(u)[j]; }

__device__ __forceinline__ void lds_store4(__bf16* p, float a, float b, float c, float d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}
__device__ __forceinline__ void lds_store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

__device__ __forceinline__ f32x4 mma_block(f32x4 acc, uint4 a, uint4 b, __bf16) {
    return mfma_bf16(as_bf16x8(a), as_bf16x8(b), acc);
}
__device__ __forceinline__ f32x4 mma_block(f32x4 acc, uint4 a, uint4 b, float) {
    const f32x4 av = as_f32x4(a), bv = as_f32x4(b);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma_f32(av[i], bv[i], acc);
    return acc;
}

// a lane's 16 bytes of an operand, each element scaled by the matching float of `f`
__device__ __forceinline__ uint4 scale_vec(uint4 v, const float* f, __bf16) {
    const bf16x8 e = as_bf16x8(v);
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)((float)e[j] * f[j]);
    return __builtin_bit_cast(uint4, r);
}
__device__ __forceinline__ uint4 scale_vec(uint4 v, const float* f, float) {
    const f32x4 e = as_f32x4(v);
    return __builtin_bit_cast(uint4, f32x4{e[0] * f[0], e[1] * f[1], e[2] * f[2], e[3] * f[3]});
}

__device__ __forceinline__ float dexp(double d) { return expf((float)d); }
__device__ __forceinline__ float dexp(float d) { return __expf(d); }

__host__ __device__ constexpr int tile_index(int tb, int sb) { return tb * (tb + 1) / 2 + sb; }
__host__ __device__ constexpr int offdiag_index(int tb, int sb) { return tb * (tb - 1) / 2 + sb; }

// LDS layout of the diagonal-decay walk, in bytes from the start (all offsets 16-aligned).
template <typename T, int N, int P>
struct DiagLayout {
    using CT = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
    static constexpr int KB = Traits<T>::kKBlock;
    static constexpr int PADE = Traits<T>::kPad;
    int Q, QK, QP, NP, NT;
    bool raw;
    size_t xt, bt, ht, cc, cf, bu, cum, beta, el, sl, braw, craw, part, total;
    __host__ __device__ DiagLayout(int q) {
        Q = q;
        QK = (q + KB - 1) / KB * KB;
        QP = QK + PADE;
        NP = N + PADE;
        NT = q / 16;
        size_t o = 0;
        auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 15) / 16 * 16; return r; };
        xt = take((size_t)P * QP * sizeof(T));        // x^T            [P][QP]
        bt = take((size_t)N * QP * sizeof(T));        // (w o B)^T      [N][QP]
        ht = take((size_t)P * NP * sizeof(T));        // H^T            [P][NP]
        cc = take((size_t)QK * NP * sizeof(T));       // C o exp(cum)   [QK][NP]
        cf = take((size_t)QK * NP * sizeof(T));       // C o f          [QK][NP]
        bu = take((size_t)QK * NP * sizeof(T));       // B o u          [QK][NP]
        cum = take((size_t)QK * N * sizeof(CT));      // running sums   [QK][N]
        beta = take((size_t)(NT * (NT - 1) / 2 + 1) * N * sizeof(float));
        el = take((size_t)N * sizeof(float));
        sl = take((size_t)(NT * (NT + 1) / 2) * 256 * sizeof(float));  // masked score tiles
        part = take((size_t)(kThreads / N + 1) * N * sizeof(CT));        // scan partial sums
        // raw B and C rows for the exact diagonal tiles when they fit in LDS next to the rest
        // (otherwise those tiles read them from global memory)
        braw = craw = 0;
        raw = o + 2 * (((size_t)QK * NP * sizeof(T) + 15) / 16 * 16) <= kMaxLds;
        if (raw) {
            braw = take((size_t)QK * NP * sizeof(T));   // B    [QK][NP]
            craw = take((size_t)QK * NP * sizeof(T));   // C    [QK][NP]
        }
        total = o;
    }
};

template <typename T, int N, int P>
__global__ void __launch_bounds__(kThreads) walk_diag_kernel(WalkParams prm) {
    using TR = Traits<T>;
    using L = DiagLayout<T, N, P>;
    using CT = typename L::CT;
    constexpr int KB = TR::kKBlock;
    constexpr int VE = TR::kVec;
    constexpr int PB = P / 16;
    constexpr int NB = N / 16;
    constexpr int NTILE = NB * PB;
    constexpr int TPW = (NTILE + kWaves - 1) / kWaves;

    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, prm.batch * H);
    if (unit < 0) return;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
    // (the wave index made wave-uniform, so that the per-wave item loops run as scalar loops)
    const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, lg = lane / 16;
    const int koff = (KB / 4) * lg;
    const L lay(prm.chunk);
    const int Q = lay.Q, QK = lay.QK, QP = lay.QP, NP = lay.NP, nt = lay.NT;

    extern __shared__ __align__(16) unsigned char smem[];
    T* Xt = reinterpret_cast<T*>(smem + lay.xt);
    T* Bt = reinterpret_cast<T*>(smem + lay.bt);
    T* Ht = reinterpret_cast<T*>(smem + lay.ht);
    T* Cc = reinterpret_cast<T*>(smem + lay.cc);
    T* Cf = reinterpret_cast<T*>(smem + lay.cf);
    T* Bu = reinterpret_cast<T*>(smem + lay.bu);
    CT* cum = reinterpret_cast<CT*>(smem + lay.cum);
    CT* part = reinterpret_cast<CT*>(smem + lay.part);
    T* Braw = reinterpret_cast<T*>(smem + lay.braw);
    T* Craw = reinterpret_cast<T*>(smem + lay.craw);
    const bool kRawLds = lay.raw;
    float* beta = reinterpret_cast<float*>(smem + lay.beta);
    float* el = reinterpret_cast<float*>(smem + lay.el);
    float* Sl = reinterpret_cast<float*>(smem + lay.sl);

    const T* xg = static_cast<const T*>(prm.x);
    const T* Bg = static_cast<const T*>(prm.Bm);
    const T* Cg = static_cast<const T*>(prm.Cm);
    T* yg = static_cast<T*>(prm.y);
    const uint4 zero = {0u, 0u, 0u, 0u};
    const float dskip = prm.D ? prm.D[h] : 0.f;

    // ---- state registers (tiles (nb, pb) dealt round-robin to the waves)
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
                lds_store4(Ht + (16 * pb + l16) * NP + 16 * nb + 4 * lg, hs[j][0], hs[j][1], hs[j][2], hs[j][3]);
            }
        }
    };
    write_state_lds();

    const int nch = (int)((sq.len + Q - 1) / Q);
    for (int c = 0; c < nch; ++c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, sq.len - t0);
        __syncthreads();  // previous chunk done with every LDS buffer

        // ---- 1. log a into LDS, then running sums down each state column (past the end: 0):
        //         kThreads / N groups of consecutive tokens per column, each summed by one
        //         thread, then every group offset by the totals of the groups before it
        for (int i = tid; i < QK * N; i += kThreads) {
            const int t = i / N, n = i % N;
            cum[i] = t < len ? (CT)prm.log_a[((sq.row0 + t0 + t) * H + h) * N + n] : (CT)0;
        }
        __syncthreads();
        {
            constexpr int NG = kThreads / N;  // token groups per column
            const int n = tid % N, grp = tid / N, per = (QK + NG - 1) / NG;
            const int ta = min(QK, grp * per), tz = min(QK, ta + per);
            CT run = 0;
            for (int t = ta; t < tz; ++t) {
                run += cum[t * N + n];
                cum[t * N + n] = run;
            }
            part[grp * N + n] = run;
            __syncthreads();
            CT off = 0;
            for (int q = 0; q < grp; ++q) off += part[q * N + n];
            for (int t = ta; t < tz; ++t) cum[t * N + n] += off;
        }
        __syncthreads();

        // ---- 2. factor tables and scaled operands
        for (int n = tid; n < N; n += kThreads) el[n] = dexp(cum[(Q - 1) * N + n]);
        for (int i = tid; i < (nt * (nt - 1) / 2) * N; i += kThreads) {
            const int p = i / N, n = i % N;
            int tb = 1;
            while (offdiag_index(tb + 1, 0) <= p) ++tb;
            const int sb = p - offdiag_index(tb, 0);
            beta[i] = dexp(cum[(16 * tb) * N + n] - cum[(16 * sb + 15) * N + n]);
        }
        for (int item = tid; item < QK * (N / VE); item += kThreads) {
            const int t = item / (N / VE), cc = item % (N / VE);
            const bool ok = t < len;
            const uint4 cv = ok ? ld16(Cg + ((sq.row0 + t0 + t) * G + g) * N + cc * VE) : zero;
            const uint4 bv = ok ? ld16(Bg + ((sq.row0 + t0 + t) * G + g) * N + cc * VE) : zero;
            const int a = t & ~15, e = t | 15;
            float fe[VE], ff_[VE], fu[VE];
#pragma unroll
            for (int j = 0; j < VE; ++j) {
                const int n = cc * VE + j;
                const CT ct = cum[t * N + n];
                fe[j] = dexp(ct);
                ff_[j] = dexp(ct - cum[a * N + n]);
                fu[j] = dexp(cum[min(e, QK - 1) * N + n] - ct);
            }
            st16(Cc + t * NP + cc * VE, scale_vec(cv, fe, T()));
            st16(Cf + t * NP + cc * VE, scale_vec(cv, ff_, T()));
            st16(Bu + t * NP + cc * VE, scale_vec(bv, fu, T()));
            if (kRawLds) {
                st16(Craw + t * NP + cc * VE, cv);
                st16(Braw + t * NP + cc * VE, bv);
            }
        }
        // x^T and (w o B)^T, four tokens per thread and 16-byte global loads
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
                lds_store4(Xt + (cc * VE + j) * QP + 4 * rg, (float)vec_elem<T>(u[0], j), (float)vec_elem<T>(u[1], j),
                           (float)vec_elem<T>(u[2], j), (float)vec_elem<T>(u[3], j));
        }
        for (int item = tid; item < (QK / 4) * (N / VE); item += kThreads) {
            const int rg = item / (N / VE), cc = item % (N / VE);
            uint4 u[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 4 * rg + k;
                u[k] = r < len ? ld16(Bg + ((sq.row0 + t0 + r) * G + g) * N + cc * VE) : zero;
            }
#pragma unroll
            for (int j = 0; j < VE; ++j) {
                const int n = cc * VE + j;
                const CT cl = cum[(Q - 1) * N + n];
                float w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) w[k] = dexp(cl - cum[(4 * rg + k) * N + n]);
                lds_store4(Bt + n * QP + 4 * rg, w[0] * (float)vec_elem<T>(u[0], j), w[1] * (float)vec_elem<T>(u[1], j),
                           w[2] * (float)vec_elem<T>(u[2], j), w[3] * (float)vec_elem<T>(u[3], j));
            }
        }
        __syncthreads();

        // ---- 3. masked score tiles S^T[s][t] (s block sb <= t block tb), fp32 in LDS,
        //         accumulator order: lane l holds rows 4(l/16)+i, column l%16
        // (the costly diagonal tiles first, one per wave, then the others round-robin)
        const int ntiles = nt * (nt + 1) / 2;
        for (int ord = wave; ord < ntiles; ord += kWaves) {
            int tb, sb;
            if (ord < nt) {
                tb = sb = ord;
            } else {
                const int o = ord - nt;  // o-th off-diagonal tile in row order
                tb = 1;
                while (offdiag_index(tb + 1, 0) <= o) ++tb;
                sb = o - offdiag_index(tb, 0);
            }
            const int idx = tile_index(tb, sb);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (sb < tb) {
                const float* bet = beta + offdiag_index(tb, sb) * N;
                const int s = 16 * sb + l16, t = 16 * tb + l16;
#pragma unroll
                for (int kb = 0; kb < N / KB; ++kb) {
                    const int k0 = kb * KB + koff;
                    const uint4 av = ld16(Bu + s * NP + k0);
                    const uint4 cv = scale_vec(ld16(Cf + t * NP + k0), bet + k0, T());
                    acc = mma_block(acc, av, cv, T());
                }
            } else {
                const int t = 16 * tb + l16;
                // exact: S^T[s][t] = sum_n B_sn C_tn exp(cum_tn - cum_sn), s <= t; raw B and C
                // rows come from global memory (the chunk's lines are still in cache)
                // (raw rows from LDS for 2-byte types; rows past the end are zeros there)
                for (int n = 0; n < N; ++n) {
                    const CT ct = cum[t * N + n];
                    const float craw =
                        kRawLds ? (float)Craw[t * NP + n]
                                : (float)Cg[((sq.row0 + t0 + min(t, len - 1)) * G + g) * N + n] * (t < len ? 1.f : 0.f);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = 16 * sb + 4 * lg + i;
                        const bool causal = s <= t && s < len;
                        const float braw = !causal ? 0.f
                                           : kRawLds ? (float)Braw[s * NP + n]
                                                     : (float)Bg[((sq.row0 + t0 + s) * G + g) * N + n];
                        const CT d = causal ? (CT)(ct - cum[s * N + n]) : (CT)0;
                        acc[i] += craw * braw * dexp(d);
                    }
                }
            }
            *reinterpret_cast<f32x4*>(Sl + idx * 256 + lane * 4) = acc;
        }
        __syncthreads();

        // ---- 4. outputs: carried state (C o exp(cum)) H_{k-1}, plus masked scores times x
        for (int tb = wave; tb < nt; tb += kWaves) {
            const int tl = 16 * tb + l16;
            const bool tvalid = tl < len;
            const int64_t trow = sq.row0 + t0 + tl;
            f32x4 acc[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < N / KB; ++kb) {
                const uint4 cv = ld16(Cc + tl * NP + kb * KB + koff);
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
                    acc[pb] = mma_block(acc[pb], ld16(Ht + (16 * pb + l16) * NP + kb * KB + koff), cv, T());
            }
            auto tile = [&](int sb) -> f32x4 {
                return *reinterpret_cast<const f32x4*>(Sl + tile_index(tb, sb) * 256 + lane * 4);
            };
            if constexpr (std::is_same<T, __bf16>::value) {
                for (int k = 0; 2 * k <= tb; ++k) {
                    const f32x4 m0 = tile(2 * k);
                    const f32x4 m1 = (2 * k + 1 <= tb) ? tile(2 * k + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
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
                    const f32x4 m = tile(sb);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        const f32x4 xa = as_f32x4(ld16(Xt + (16 * pb + l16) * QP + 16 * sb + 4 * lg));
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[pb] = mfma_f32(xa[i], m[i], acc[pb]);
                    }
                }
            }
            if (prm.D) {
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[pb][i] += dskip * (float)Xt[(16 * pb + 4 * lg + i) * QP + tl];
            }
            if (tvalid) {
                T* yr = yg + (trow * H + h) * P + 4 * lg;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) store4(yr + 16 * pb, acc[pb][0], acc[pb][1], acc[pb][2], acc[pb][3]);
            }
        }

        // ---- 5. state: H_k[n,:] = exp(cum_last,n) H_{k-1}[n,:] + (w o B)^T X
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                f32x4 a = hs[j];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] *= el[16 * nb + 4 * lg + i];
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
// walk_diag_pipe_kernel: the same walk for bf16 inputs and 64-token chunks, pipelined: the
// next chunk's log a, B, C and x rows are loaded into registers while the current chunk is
// computed and staged into LDS once it is done, so no phase waits on global memory; every
// operand (raw B and C included) is read from LDS.  The running sums are kept in rows padded
// to N + 4 floats so that 16 rows read at once fall on distinct banks.
constexpr int kDiagQ = 64;
constexpr int kDiagWaves = 8;
// bound (natural log) on each of the two factors a diagonal score tile splits into.  Both bf16
// and fp32 reach e^88.7 and e^-87.3 (normal range), so exp(+-80) times a B or C entry stays finite
// and normal for entries of magnitude 1e-3 .. 6e3 (a smaller entry's factor can flush to zero:
// an absolute error under 1e-3 times the other operand, below that term's bf16 rounding at
// typical magnitudes).  With the split taken halfway (in value)
// through a block's running sums, a state dimension splits when its decay over the block is at
// most 2 kSplitMax; the others take exact exponentials.  (At e^64 the multiscale workload sent
// 1.6 groups of four dimensions per block to the exact terms, at e^80 0.85: walk 84-86 -> 82 us.)
constexpr float kSplitMax = 80.f;
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kSplitMax2 = kSplitMax * kLog2eD;  // the same bound in log2 units
// 2^x on the hardware unit (v_exp_f32); results below the normal range are not kept, which only
// affects factors under 2^-126.
__device__ __forceinline__ float dexp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kDiagThreads = kDiagWaves * kWave;

// An MFMA operand of a row-major [token][col] bf16 tile in LDS, contracting over tokens, with
// the gfx950 transposing read ds_read_b64_tr_b16 (a 16-lane group whose lane 4r + q points at
// row r, columns 4q .. 4q + 3 returns in lane i column i of those four rows): lane (g, i)
// receives tile[32 k + tok(g, j)][col0 + i], j = 0..7, with tok(g, j) = 4g + j, 16 + 4g + j - 4
// (KPERM, the row order of two stacked accumulator tiles) or 8g + j (natural order).
template <bool KPERM>
__device__ __forceinline__ bf16x8 x_frag(const __bf16* tile, int stride, int col0, int k, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int g = lane / 16, r = (lane % 16) / 4, q = lane % 4;
    const int row0 = KPERM ? 32 * k + 4 * g + r : 32 * k + 8 * g + r;
    const int row1 = KPERM ? row0 + 16 : row0 + 4;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + row0 * stride + col0 + 4 * q));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + row1 * stride + col0 + 4 * q));
    const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// A 16x16x16 MFMA operand contracting over the 16 rows row0 .. row0 + 15 of a row-major bf16 tile in
// LDS: lane (g, i) receives tile[row0 + 4g + j][col0 + i], j = 0..3 (one transposing read).
__device__ __forceinline__ short __attribute__((ext_vector_type(4))) tr16(const __bf16* tile, int stride, int row0,
                                                                         int col0, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int g = lane / 16, r = (lane % 16) / 4, q = lane % 4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + (row0 + 4 * g + r) * stride + col0 + 4 * q));
}

template <int N, int P>
struct DiagPipeLayout {
    static constexpr int Q = kDiagQ, NT = Q / 16, QP = Q + 8, NP = N + 8, CS = N + 4;
    // x staged row-major with rows P + 16 elements apart: eight consecutive rows then start on
    // distinct banks for the transposing reads of its MFMA operands
    static constexpr int XS = P + 16;
    static constexpr int NOFF = NT * (NT - 1) / 2;
    // offsets in bytes
    static constexpr size_t xt = 0;                                   // x            [Q][XS] bf16
    static constexpr size_t ht = xt + (size_t)Q * XS * 2;            // H^T          [P][NP] bf16
    static constexpr size_t cc = ht + (size_t)P * NP * 2;            // C o exp(cum) [Q][NP] bf16
    static constexpr size_t cf = cc + (size_t)Q * NP * 2;            // C o f        [Q][NP] bf16
    static constexpr size_t bu = cf + (size_t)Q * NP * 2;            // B o u        [Q][NP] bf16
    static constexpr size_t braw = bu + (size_t)Q * NP * 2;          // B            [Q][NP] bf16
    static constexpr size_t craw = braw + (size_t)Q * NP * 2;        // C            [Q][NP] bf16
    static constexpr size_t cum = craw + (size_t)Q * NP * 2;         // running sums [Q][CS] f32
    static constexpr size_t part = cum + (size_t)Q * CS * 4;         // scan partials [threads/N][N]
    static constexpr size_t beta = part + (size_t)kDiagThreads * 4;  // [NOFF][N]
    static constexpr size_t el = beta + (size_t)(NOFF + 1) * N * 4;  // [NT][N] decay over each block
    // score tiles [NT(NT+1)/2][256], then the second state-dimension half of each diagonal tile
    static constexpr size_t sl = el + (size_t)NT * N * 4;
    static constexpr size_t total = sl + (size_t)(NT * (NT + 1) / 2 + NT) * 256 * 4;
};

// segments of a diagonal walk whose states each walk workgroup chains itself (a workgroup of the
// last segment reads kDiagChainMax - 1 local states of N x P floats); more go through a prefix launch
constexpr int kDiagChainMax = 4;

// DT: the discretisation front-end (prm.dt): log a = -softplus(dt + bias) exp(A_log[h, n]) is
// formed as each chunk is staged, and with prm.scale_input the staged B rows carry the input
// scale softplus(dt + bias) (B-bar = Delta B: B only ever enters as the key/input side).
template <int N, int P, bool DT = false>
__global__ void __launch_bounds__(kDiagThreads) walk_diag_pipe_kernel(WalkParams prm) {
    constexpr int kThreads = kDiagThreads, kWaves = kDiagWaves;  // (this kernel's own workgroup)
    using L = DiagPipeLayout<N, P>;
    constexpr int Q = L::Q, NT = L::NT, NP = L::NP, CS = L::CS, XS = L::XS;
    constexpr int PB = P / 16, NB = N / 16, NTILE = NB * PB, TPW = (NTILE + kWaves - 1) / kWaves;
    // 16-byte pieces per chunk of log a, of B (and of C) and of x, and per thread (rounded up;
    // the pieces past the total are skipped, which is uniform over a wave)
    constexpr int LAT = Q * N / 4, BCT = Q * N / 8, XT = Q * P / 8;
    constexpr int LAI = (LAT + kThreads - 1) / kThreads, BCI = (BCT + kThreads - 1) / kThreads;
    constexpr int XI = (XT + kThreads - 1) / kThreads;

    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen;
    const int64_t units = prm.batch * H;
    const int64_t work = xcd_work_index(blockIdx.x, prm.per_xcd, prm.nseg * units);
    if (work < 0) return;
    const int seg = (int)(work / units);
    const int64_t unit = work % units;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    // (the wave index made wave-uniform, so that the per-wave item loops run as scalar loops)
    const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, lg = lane / 16;
    const SeqSpan sq = seq_span(prm.seq_off, b, Tn, prm.total);
    // (a packed sequence: its own chunk count; it is never segmented)
    const int nchunks = prm.seq_off ? (int)((sq.len + Q - 1) / Q) : prm.nchunks;
    const int c0 = seg * prm.seg_chunks, c1 = min(c0 + prm.seg_chunks, nchunks);
    const int64_t sidx = seg * units + unit;  // (segment, unit) index of the segment buffers
    if (c1 <= c0) {
        // an empty packed sequence: its final state is its initial state
        if (prm.final_state)
            for (int i = tid; i < N * P; i += kThreads)
                prm.final_state[unit * N * P + i] = prm.init ? prm.init[unit * N * P + i] : 0.f;
        return;
    }

    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Xr = reinterpret_cast<__bf16*>(smem + L::xt);
    __bf16* Ht = reinterpret_cast<__bf16*>(smem + L::ht);
    __bf16* Cc = reinterpret_cast<__bf16*>(smem + L::cc);
    __bf16* Cf = reinterpret_cast<__bf16*>(smem + L::cf);
    __bf16* Bu = reinterpret_cast<__bf16*>(smem + L::bu);
    __bf16* Braw = reinterpret_cast<__bf16*>(smem + L::braw);
    __bf16* Craw = reinterpret_cast<__bf16*>(smem + L::craw);
    float* cum = reinterpret_cast<float*>(smem + L::cum);
    float* part = reinterpret_cast<float*>(smem + L::part);
    float* beta = reinterpret_cast<float*>(smem + L::beta);
    float* el = reinterpret_cast<float*>(smem + L::el);
    float* Sl = reinterpret_cast<float*>(smem + L::sl);

    const float* lag = prm.log_a;
    const float* dtg = prm.dt;
    // (DT) this thread's log a factors -exp(A_log[h, n]) log2(e) for its 4 state dims: the la
    // pieces it stages all sit at n = 4 (tid % (N / 4)), since the thread count is a multiple
    // of N / 4
    static_assert(kThreads % (N / 4) == 0, "la pieces of a thread share their state dims");
    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
    float dt_b = 0.f;
    if (DT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a4[j] = -expf(prm.A_log[h * N + 4 * (tid % (N / 4)) + j]) * kLog2eD;
        dt_b = prm.dt_bias ? prm.dt_bias[h] : 0.f;
    }
    const __bf16* xg = static_cast<const __bf16*>(prm.x);
    const __bf16* Bg = static_cast<const __bf16*>(prm.Bm);
    const __bf16* Cg = static_cast<const __bf16*>(prm.Cm);
    __bf16* yg = static_cast<__bf16*>(prm.y);
    const uint4 zero = {0u, 0u, 0u, 0u};
    const float dskip = prm.D ? prm.D[h] : 0.f;
    auto chunk_len = [&](int c) { return (int)min((int64_t)Q, sq.len - (int64_t)c * Q); };

    // ---- prefetch registers: one chunk of log a, B, C and x rows (rows clamped into the
    //      sequence; staged as zeros past its end)
    uint4 rla[LAI], rb[BCI], rc[BCI], rx[XI];
    // (DT) dt of token `lane` of the chunk (Q = 64 tokens, one per lane): each lane forms that
    // token's step size once, and the threads staging a row take it from that lane
    static_assert(!DT || Q == kWave, "one token per lane");
    float rdt = 0.f;
    auto load_chunk = [&](int c) {
        const int64_t t0 = (int64_t)c * Q;
        const int last = chunk_len(c) - 1;
        if (DT) rdt = dtg[(sq.row0 + t0 + min(lane, last)) * H + h];
#pragma unroll
        for (int m = 0; m < LAI; ++m) {
            const int id = tid + kThreads * m, t = min(id / (N / 4), last), c4 = id % (N / 4);
            if (!DT && id < LAT) rla[m] = ld16(lag + ((sq.row0 + t0 + t) * H + h) * N + 4 * c4);
        }
#pragma unroll
        for (int m = 0; m < BCI; ++m) {
            const int id = tid + kThreads * m, t = min(id / (N / 8), last), c8 = id % (N / 8);
            const int64_t off = ((sq.row0 + t0 + t) * G + g) * N + 8 * c8;
            if (id < BCT) {
                rb[m] = ld16(Bg + off);
                rc[m] = ld16(Cg + off);
            }
        }
#pragma unroll
        for (int m = 0; m < XI; ++m) {
            const int id = tid + kThreads * m, t = min(id / (P / 8), last), c8 = id % (P / 8);
            if (id < XT) rx[m] = ld16(xg + ((sq.row0 + t0 + t) * H + h) * P + 8 * c8);
        }
    };
    auto stage_chunk = [&](int c) {
        const int len = chunk_len(c);
        const float delta = DT ? softplus_hw(rdt + dt_b) : 0.f;  // step size of token `lane`
#pragma unroll
        for (int m = 0; m < LAI; ++m) {
            const int id = tid + kThreads * m, t = id / (N / 4), c4 = id % (N / 4);
            // (the shuffle outside the branch: every lane of the wave takes part)
            const float dt_row = DT ? __shfl(delta, t % Q, kWave) : 0.f;
            // log a in log2 units, so that every factor below is one exp2
            if (id < LAT) {
                const f32x4 v = DT ? dt_row * a4 : __builtin_bit_cast(f32x4, rla[m]) * kLog2eD;
                st16(cum + t * CS + 4 * c4, t < len ? __builtin_bit_cast(uint4, v) : zero);
            }
        }
#pragma unroll
        for (int m = 0; m < BCI; ++m) {
            const int id = tid + kThreads * m, t = id / (N / 8), c8 = id % (N / 8);
            const float dt_row = DT ? __shfl(delta, t % Q, kWave) : 0.f;
            if (id < BCT) {
                uint4 bv = rb[m];
                if (DT && prm.scale_input) {
                    bf16x8 sv = as_bf16x8(bv);
#pragma unroll
                    for (int j = 0; j < 8; ++j) sv[j] = (__bf16)((float)sv[j] * dt_row);
                    bv = __builtin_bit_cast(uint4, sv);
                }
                st16(Braw + t * NP + 8 * c8, t < len ? bv : zero);
                st16(Craw + t * NP + 8 * c8, t < len ? rc[m] : zero);
            }
        }
#pragma unroll
        for (int m = 0; m < XI; ++m) {
            const int id = tid + kThreads * m, t = id / (P / 8), c8 = id % (P / 8);
            if (id < XT) st16(Xr + t * XS + 8 * c8, t < len ? rx[m] : zero);
        }
    };

    // ---- state registers (tiles (nb, pb) dealt round-robin to the waves)
    // The state entering the segment: the caller's initial state for the first one; for a later
    // one either the prefix launch's chained state (seg_init), or, with seg_init null, the chain
    // h <- exp2(decay_j) o h + state_j over the segments j < seg run here from the caller's initial
    // state (per state dimension n; local states and log2 decays from seg_state_diag_kernel).
    f32x4 hs[TPW];
    const bool chain = prm.nseg > 1 && !prm.seg_init;
    const float* init = prm.nseg > 1 && !chain ? prm.seg_init + sidx * N * P
                                               : (prm.init ? prm.init + unit * N * P : nullptr);
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        hs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = wave + kWaves * j;
        if (tile < NTILE && init) {
            const int nb = tile / PB, pb = tile % PB;
            const float* src = init + (16 * nb + 4 * lg) * P + 16 * pb + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) hs[j][i] = src[i * P];
        }
    }
    // (the chain's loads issued here, with the first chunk's; its arithmetic once they are in)
    constexpr int CH = kDiagChainMax - 1;
    f32x4 cst[CH][TPW], cdc[CH][TPW];
    if (chain) {
#pragma unroll
        for (int js = 0; js < CH; ++js)
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int tile = wave + kWaves * j;
                cst[js][j] = cdc[js][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (js < seg && tile < NTILE) {
                    const int nb = tile / PB, pb = tile % PB, n = 16 * nb + 4 * lg;
                    const float* src = prm.seg_state + (js * units + unit) * N * P + n * P + 16 * pb + l16;
                    const float* dc = prm.seg_decay + (js * units + unit) * N + n;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        cst[js][j][i] = src[i * P];
                        cdc[js][j][i] = dc[i];
                    }
                }
            }
    }
    auto chain_states = [&]() {
#pragma unroll
        for (int js = 0; js < CH; ++js)
#pragma unroll
            for (int j = 0; j < TPW; ++j)
                if (js < seg)
#pragma unroll
                    for (int i = 0; i < 4; ++i) hs[j][i] = exp2f(cdc[js][j][i]) * hs[j][i] + cst[js][j][i];
    };
    auto write_state_lds = [&]() {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                lds_store4(Ht + (16 * pb + l16) * NP + 16 * nb + 4 * lg, hs[j][0], hs[j][1], hs[j][2], hs[j][3]);
            }
        }
    };

    load_chunk(c0);
    stage_chunk(c0);
    if (chain) chain_states();
    write_state_lds();
    load_chunk(min(c0 + 1, c1 - 1));

    for (int c = c0; c < c1; ++c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = chunk_len(c);
        __syncthreads();  // chunk c staged; everything of chunk c-1 done

        // ---- 1. running sums down each state column (kThreads / N token groups per column)
        {
            // (each thread's PER values read at once and kept in registers; the partial sums of the
            // groups before it read at once, unrolled and masked)
            constexpr int NGR = kThreads / N, PER = Q / NGR;
            const int n = tid % N, grp = tid / N;
            float v[PER];
#pragma unroll
            for (int k = 0; k < PER; ++k) v[k] = cum[(grp * PER + k) * CS + n];
#pragma unroll
            for (int k = 1; k < PER; ++k) v[k] += v[k - 1];
            part[grp * N + n] = v[PER - 1];
            __syncthreads();
            float pv[NGR - 1];
#pragma unroll
            for (int q = 0; q < NGR - 1; ++q) pv[q] = part[q * N + n];
            float off = 0.f;
#pragma unroll
            for (int q = 0; q < NGR - 1; ++q) off += q < grp ? pv[q] : 0.f;
#pragma unroll
            for (int k = 0; k < PER; ++k) cum[(grp * PER + k) * CS + n] = v[k] + off;
        }
        __syncthreads();

        // ---- 2. factor tables and scaled operands (all from LDS)
        // decay over each 16-token block per state dimension: E_b = exp(cum_end(b) - cum_end(b-1))
        for (int i = tid; i < NT * N; i += kThreads) {
            const int bk = i / N, n = i % N;
            el[i] = dexp2(cum[(16 * bk + 15) * CS + n] - (bk > 0 ? cum[(16 * bk - 1) * CS + n] : 0.f));
        }
        for (int i = tid; i < L::NOFF * N; i += kThreads) {
            const int p = i / N, n = i % N;
            int tb = 1;
            while (offdiag_index(tb + 1, 0) <= p) ++tb;
            const int sb = p - offdiag_index(tb, 0);
            beta[i] = dexp2(cum[(16 * tb) * CS + n] - cum[(16 * sb + 15) * CS + n]);
        }
        for (int item = tid; item < Q * (N / 8); item += kThreads) {
            const int t = item / (N / 8), c8 = item % (N / 8);
            const int a = t & ~15, e = t | 15;
            // (C o exp(cum), C o f for the output side; B o u, which also feeds the state update)
            const f32x4 ct0 = *reinterpret_cast<const f32x4*>(cum + t * CS + 8 * c8);
            const f32x4 ct1 = *reinterpret_cast<const f32x4*>(cum + t * CS + 8 * c8 + 4);
            const f32x4 ca0 = *reinterpret_cast<const f32x4*>(cum + a * CS + 8 * c8);
            const f32x4 ca1 = *reinterpret_cast<const f32x4*>(cum + a * CS + 8 * c8 + 4);
            const f32x4 ce0 = *reinterpret_cast<const f32x4*>(cum + e * CS + 8 * c8);
            const f32x4 ce1 = *reinterpret_cast<const f32x4*>(cum + e * CS + 8 * c8 + 4);
            const bf16x8 cv = as_bf16x8(ld16(Craw + t * NP + 8 * c8));
            const bf16x8 bv = as_bf16x8(ld16(Braw + t * NP + 8 * c8));
            bf16x8 vcc, vcf, vbu;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float ct = j < 4 ? ct0[j] : ct1[j - 4];
                const float ca = j < 4 ? ca0[j] : ca1[j - 4];
                const float ce = j < 4 ? ce0[j] : ce1[j - 4];
                vcc[j] = (__bf16)((float)cv[j] * dexp2(ct));
                vcf[j] = (__bf16)((float)cv[j] * dexp2(ct - ca));
                vbu[j] = (__bf16)((float)bv[j] * dexp2(ce - ct));
            }
            *reinterpret_cast<bf16x8*>(Cc + t * NP + 8 * c8) = vcc;
            *reinterpret_cast<bf16x8*>(Cf + t * NP + 8 * c8) = vcf;
            *reinterpret_cast<bf16x8*>(Bu + t * NP + 8 * c8) = vbu;
        }
        __syncthreads();

        // ---- 3. masked score tiles S^T[s][t] (s block sb <= t block tb), fp32 in LDS, in
        //         accumulator order (lane l holds rows 4(l/16)+i, column l%16); the costly
        //         diagonal tiles first, one per wave
        constexpr int NTILES = NT * (NT + 1) / 2;
        // items: the two state-dimension halves of every diagonal tile (costly: one wave each),
        // then the off-diagonal tiles
        for (int item = wave; item < 2 * NT + L::NOFF; item += kWaves) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            float* dst;
            if (item >= 2 * NT) {
                const int o = item - 2 * NT;
                int tb = 1;
                while (offdiag_index(tb + 1, 0) <= o) ++tb;
                const int sb = o - offdiag_index(tb, 0);
                const float* bet = beta + offdiag_index(tb, sb) * N;
                const int s = 16 * sb + l16, t = 16 * tb + l16;
#pragma unroll
                for (int kb = 0; kb < N / 32; ++kb) {
                    const int k0 = 32 * kb + 8 * lg;
                    float bf[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) bf[j] = bet[k0 + j];
                    const uint4 av = ld16(Bu + s * NP + k0);
                    const uint4 cv = scale_vec(ld16(Cf + t * NP + k0), bf, __bf16());
                    acc = mfma_bf16(as_bf16x8(av), as_bf16x8(cv), acc);
                }
                dst = Sl + tile_index(tb, sb) * 256;
            } else {
                // Diagonal tile, S^T[s][t] = sum_n B_sn C_tn exp(cum_tn - cum_sn) for s <= t.  For
                // a state dimension whose decay D over the block is at most 2 kSplitMax, the
                // exponential splits at m_n = (cum_an + cum_en) / 2 (a, e the block's first and
                // last token) into exp(cum_tn - m_n) and exp(m_n - cum_sn), each within
                // e^(+-D/2), and the sum over those dimensions is one MFMA contraction (wave
                // nh = 0).  (Above the diagonal the two factors can multiply past the fp32 range;
                // those entries are dropped by a select.)  The other dimensions take exact
                // exponentials, split over the two waves by halves of the state dimension.
                const int tb = item % NT, nh = item / NT, a = 16 * tb;
                const int t = a + l16;
                bool causal[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) causal[i] = 4 * lg + i <= l16;
                // dimensions too fast to split in this block (bit n)
                uint64_t fast = 0;
#pragma unroll
                for (int q = 0; q < (N + kWave - 1) / kWave; ++q) {
                    const int n = min(q * kWave + lane, N - 1);
                    const float dec = cum[a * CS + n] - cum[(a + 15) * CS + n];
                    const uint64_t bits = __ballot(dec > 2.f * kSplitMax2);
                    constexpr uint64_t kRowMask = N >= kWave ? ~0ull : (1ull << (N % kWave)) - 1;
                    fast |= (bits & kRowMask) << (q * kWave);
                }
                if (nh == 0) {
#pragma unroll
                    for (int kb = 0; kb < N / 32; ++kb) {
                        const int k0 = 32 * kb + 8 * lg;
                        const f32x4 ca0 = *reinterpret_cast<const f32x4*>(cum + a * CS + k0);
                        const f32x4 ca1 = *reinterpret_cast<const f32x4*>(cum + a * CS + k0 + 4);
                        const f32x4 ce0 = *reinterpret_cast<const f32x4*>(cum + (a + 15) * CS + k0);
                        const f32x4 ce1 = *reinterpret_cast<const f32x4*>(cum + (a + 15) * CS + k0 + 4);
                        const f32x4 cs0 = *reinterpret_cast<const f32x4*>(cum + t * CS + k0);
                        const f32x4 cs1 = *reinterpret_cast<const f32x4*>(cum + t * CS + k0 + 4);
                        const bf16x8 bv = as_bf16x8(ld16(Braw + t * NP + k0));
                        const bf16x8 cv = as_bf16x8(ld16(Craw + t * NP + k0));
                        bf16x8 bo, co;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float cm = 0.5f * ((j < 4 ? ca0[j] : ca1[j - 4]) + (j < 4 ? ce0[j] : ce1[j - 4]));
                            const float cl = j < 4 ? cs0[j] : cs1[j - 4];  // cum of this lane's row
                            const bool split = !((fast >> (k0 + j)) & 1);
                            bo[j] = (__bf16)(split ? (float)bv[j] * dexp2(cm - cl) : 0.f);  // rows s
                            co[j] = (__bf16)(split ? (float)cv[j] * dexp2(cl - cm) : 0.f);  // cols t
                        }
                        acc = mfma_bf16(bo, co, acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = causal[i] ? acc[i] : 0.f;
                }
                // exact part: groups of 4 dimensions holding a fast one, alternately to the two waves,
                // two groups at a time with every LDS read of both issued before the arithmetic (the
                // second of a last odd group is group 0 with no dimension selected: it adds zeros)
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                uint32_t gmask = 0;  // this wave's groups holding a fast dimension (bit g4)
#pragma unroll
                for (int g4 = nh; g4 < N / 4; g4 += 2)
                    gmask |= (((uint32_t)(fast >> (4 * g4)) & 0xfu) != 0u ? 1u : 0u) << g4;
                while (gmask) {
                    int gsel[2];
                    uint32_t gbits[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        gsel[u] = gmask ? __builtin_ctz(gmask) : 0;
                        gbits[u] = gmask ? (uint32_t)(fast >> (4 * gsel[u])) & 0xfu : 0u;
                        gmask &= gmask - 1u;
                    }
                    f32x4 ct[2], cs[2][4];
                    bf16x4 cr[2], br[2][4];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int n = 4 * gsel[u];
                        ct[u] = *reinterpret_cast<const f32x4*>(cum + t * CS + n);
                        cr[u] = *reinterpret_cast<const bf16x4*>(Craw + t * NP + n);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int s = a + 4 * lg + i;
                            cs[u][i] = *reinterpret_cast<const f32x4*>(cum + s * CS + n);
                            br[u][i] = *reinterpret_cast<const bf16x4*>(Braw + s * NP + n);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float cm[4];  // C on the group's fast dimensions only
#pragma unroll
                        for (int j = 0; j < 4; ++j) cm[j] = ((gbits[u] >> j) & 1) ? (float)cr[u][j] : 0.f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // (the exponent is clamped at 0 so that the entries above the diagonal,
                            // dropped below, stay finite; on and below it, it is <= 0 already)
                            float sum = 0.f;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                sum = fmaf(cm[j] * (float)br[u][i][j], dexp2(fminf(ct[u][j] - cs[u][i][j], 0.f)), sum);
                            acc[i] += causal[i] ? sum : 0.f;
                        }
                    }
                }
                dst = Sl + (nh == 0 ? tile_index(tb, tb) : NTILES + tb) * 256;
            }
            *reinterpret_cast<f32x4*>(dst + lane * 4) = acc;
        }
        __syncthreads();

        // ---- 4. outputs: carried state (C o exp(cum)) H_{k-1}, plus masked scores times x;
        //         two waves per 16-token block, each with half of the head dimension
        for (int item = wave; item < 2 * NT; item += kWaves) {
            constexpr int PH = PB / 2;
            const int tb = item % NT, pb0 = (item / NT) * PH;
            const int tl = 16 * tb + l16;
            f32x4 acc[PH];
#pragma unroll
            for (int q = 0; q < PH; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < N / 32; ++kb) {
                const uint4 cv = ld16(Cc + tl * NP + 32 * kb + 8 * lg);
#pragma unroll
                for (int q = 0; q < PH; ++q)
                    acc[q] = mfma_bf16(as_bf16x8(ld16(Ht + (16 * (pb0 + q) + l16) * NP + 32 * kb + 8 * lg)),
                                       as_bf16x8(cv), acc[q]);
            }
            auto tile = [&](int sb) -> f32x4 {
                f32x4 m = *reinterpret_cast<const f32x4*>(Sl + tile_index(tb, sb) * 256 + lane * 4);
                if (sb == tb) m += *reinterpret_cast<const f32x4*>(Sl + (NTILES + tb) * 256 + lane * 4);
                return m;
            };
            for (int k = 0; 2 * k <= tb; ++k) {
                const f32x4 m0 = tile(2 * k);
                const f32x4 m1 = (2 * k + 1 <= tb) ? tile(2 * k + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
                const bf16x8 bop = {(__bf16)m0[0], (__bf16)m0[1], (__bf16)m0[2], (__bf16)m0[3],
                                    (__bf16)m1[0], (__bf16)m1[1], (__bf16)m1[2], (__bf16)m1[3]};
#pragma unroll
                for (int q = 0; q < PH; ++q)
                    acc[q] = mfma_bf16(x_frag<true>(Xr, XS, 16 * (pb0 + q), k, lane), bop, acc[q]);
            }
#pragma unroll
            for (int q = 0; q < PH; ++q) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(Xr + tl * XS + 16 * (pb0 + q) + 4 * lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[q][i] += dskip * (float)x4[i];
            }
            if (tl < len) {
                __bf16* yr = yg + ((sq.row0 + t0 + tl) * H + h) * P + 4 * lg;
#pragma unroll
                for (int q = 0; q < PH; ++q)
                    store4(yr + 16 * (pb0 + q), acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
            }
        }

        // ---- 5. state: H_k[n,:] = exp(cum_last,n) H_{k-1}[n,:] + sum_s B_sn exp(cum_last,n - cum_sn) x_s,
        //         block by block (Horner): H <- E_b o H + (B o u)_b^T X_b, the decay from each token
        //         to its block's end inside B o u and from block to block in E_b (every factor <= 1)
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                f32x4 a = hs[j];
#pragma unroll
                for (int bk = 0; bk < NT; ++bk) {
                    const f32x4 eb = *reinterpret_cast<const f32x4*>(el + bk * N + 16 * nb + 4 * lg);
                    a *= eb;
                    a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(tr16(Bu, NP, 16 * bk, 16 * nb, lane),
                                                                 tr16(Xr, XS, 16 * bk, 16 * pb, lane), a, 0, 0, 0);
                }
                hs[j] = a;
            }
        }
        __syncthreads();  // every read of chunk c's LDS data done
        write_state_lds();
        stage_chunk(c + 1 < c1 ? c + 1 : c);
        load_chunk(min(c + 2, c1 - 1));
    }

    float* fin = (c1 == nchunks && prm.final_state) ? prm.final_state + unit * N * P : nullptr;
    if (fin) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kWaves * j;
            if (tile < NTILE) {
                const int nb = tile / PB, pb = tile % PB;
                float* dst = fin + (16 * nb + 4 * lg) * P + 16 * pb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * P] = hs[j][i];
            }
        }
    }
}

// log2 weight below which exp2 is 0 in fp32 whatever its last-bit error (the smallest denormal
// is 2^-149), and the log2 of the largest input scale (the front-end's Delta) allowed for
constexpr float kVanishDiag2 = -160.f;
constexpr float kLog2ScaleMaxDiag = 64.f;

// seg_state_diag_kernel: the state-only pass of the segmented diagonal walk.  One workgroup per
// (segment, batch, head) forms the segment's local state (its final state from a zero start) as
// one sum over its tokens,
//   H_seg[n, :] = sum_s W_sn B_sn x_s^T,   W_sn = exp(decay of state row n from token s to the
//   segment's end),
// the diagonal chunk recurrence unrolled, and the segment's log2 decay per state row.  The chunks
// are taken last to first, so the decay from a chunk's end to the segment's end is the running sum
// (per row) of the chunks already done and every W_sn <= 1: the weights go onto B, (B o W)^T x is
// one bf16 MFMA contraction over the chunk's tokens, and the state registers are only ever
// accumulated into.  In a workgroup of eight waves, thread (n, part) scans log a down state column
// n over its part of the chunk's tokens (the partial sums of the parts through LDS) and forms B o W
// for those tokens; the waves split the N x P state's 16 x 16 tiles.  With the front-end every
// wave forms the chunk's step sizes, one token per lane (Q = 64), and takes those of its tokens by
// lane shuffles.  The next chunk's log a (or dt), B and x are loaded while the current one is
// computed.  Once every row's weights are below 2^-160 (2^-224 with an input scale of up to
// 2^64), where exp2 is 0 in fp32, the earlier tokens would add exact zeros and the pass stops: the
// decays it records are then below that bound too, and the prefix of segment states weighs their
// states by exp2 of them, which is 0 either way.  (The first form ran the 8-wave walk with its
// per-block factor tables: 30 us at the multiscale shape.)
constexpr int kSegDiagWaves = 8, kSegDiagThreads = kSegDiagWaves * kWave;
template <int N, int P>
struct SegDiagShape {
    static constexpr int Q = kDiagQ, PARTS = kSegDiagThreads / N, TP = Q / PARTS;
    // 16-byte pieces of B (and of x) per chunk, and per thread (rounded up; the rest skipped)
    static constexpr int BCT = Q * N / 8, XT = Q * P / 8;
    static constexpr int BCI = (BCT + kSegDiagThreads - 1) / kSegDiagThreads, XI = (XT + kSegDiagThreads - 1) / kSegDiagThreads;
    static constexpr int NS = N + 8, XS = P + 8;  // LDS row strides (elements)
    static constexpr int NTILE = (N / 16) * (P / 16), TPW = (NTILE + kSegDiagWaves - 1) / kSegDiagWaves;
    static_assert(PARTS * N == kSegDiagThreads && TP >= 1 && Q == kWave, "segment state shape");
    // B [Q][NS] bf16, B o W [Q][NS] bf16, x [Q][XS] bf16, partial sums [PARTS][N] f32
    static constexpr size_t bs = 0, bw = bs + (size_t)Q * NS * 2, xs = bw + (size_t)Q * NS * 2;
    static constexpr size_t tot = xs + (size_t)Q * XS * 2, lds_bytes = tot + (size_t)PARTS * N * 4;
};

template <int N, int P, bool DT>
__global__ void __launch_bounds__(kSegDiagThreads) seg_state_diag_kernel(WalkParams prm) {
    using S = SegDiagShape<N, P>;
    constexpr int Q = S::Q, TP = S::TP, BCI = S::BCI, XI = S::XI, NS = S::NS, XS = S::XS;
    constexpr int PB = P / 16, TPW = S::TPW, NTILE = S::NTILE;
    const int64_t H = prm.nheads, G = prm.ngroups;
    const int64_t units = prm.batch * H;
    const int64_t work = xcd_work_index(blockIdx.x, prm.per_xcd, prm.nseg * units);
    if (work < 0) return;
    const int seg = (int)(work / units);
    const int64_t unit = work % units;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n = tid % N, part = tid / N;
    const int64_t row0 = b * prm.seqlen;
    const int c0 = seg * prm.seg_chunks, c1 = min(c0 + prm.seg_chunks, prm.nchunks);
    const int64_t sidx = seg * units + unit;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Bs = reinterpret_cast<__bf16*>(smem + S::bs);
    __bf16* BWs = reinterpret_cast<__bf16*>(smem + S::bw);
    __bf16* Xs = reinterpret_cast<__bf16*>(smem + S::xs);
    float* tot = reinterpret_cast<float*>(smem + S::tot);
    const __bf16* xg = static_cast<const __bf16*>(prm.x);
    const __bf16* Bg = static_cast<const __bf16*>(prm.Bm);
    auto chunk_len = [&](int c) { return (int)min((int64_t)Q, prm.seqlen - (int64_t)c * Q); };
    // (DT) -exp(A_log[h, n]) log2(e) of this thread's state row, and the step-size bias
    const float an = DT ? -expf(prm.A_log[h * N + n]) * kLog2eD : 0.f;
    const float dtb = DT && prm.dt_bias ? prm.dt_bias[h] : 0.f;

    // prefetch registers: this thread's log a column over its tokens (with the front-end: the dt
    // of token `lane`), its pieces of B and of x (rows clamped into the sequence, staged as zeros
    // past its end)
    float la[DT ? 1 : TP];
    uint4 rb[BCI], rx[XI];
    auto load_chunk = [&](int c) {
        const int64_t t0 = (int64_t)c * Q;
        const int last = chunk_len(c) - 1;
        if (DT) {
            la[0] = prm.dt[(row0 + t0 + min(lane, last)) * H + h];
        } else {
#pragma unroll
            for (int i = 0; i < TP; ++i)
                la[i] = prm.log_a[((row0 + t0 + min(part * TP + i, last)) * H + h) * N + n];
        }
#pragma unroll
        for (int m = 0; m < BCI; ++m) {
            const int id = min(tid + kSegDiagThreads * m, S::BCT - 1), t = min(id / (N / 8), last), c8 = id % (N / 8);
            rb[m] = ld16(Bg + ((row0 + t0 + t) * G + g) * N + 8 * c8);
        }
#pragma unroll
        for (int m = 0; m < XI; ++m) {
            const int id = min(tid + kSegDiagThreads * m, S::XT - 1), t = min(id / (P / 8), last), c8 = id % (P / 8);
            rx[m] = ld16(xg + ((row0 + t0 + t) * H + h) * P + 8 * c8);
        }
    };

    f32x4 hs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) hs[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float sfx = 0.f;  // log2 decay of row n from the end of the chunk in hand to the segment's end
    // (with an input scale its B entries carry a factor of up to 2^64)
    const float vanish = kVanishDiag2 - (DT && prm.scale_input ? kLog2ScaleMaxDiag : 0.f);
    load_chunk(c1 - 1);
    for (int c = c1 - 1; c >= c0; --c) {
        const int len = chunk_len(c);
        // stage B and x (and the step size of each token)
#pragma unroll
        for (int m = 0; m < BCI; ++m) {
            const int id = tid + kSegDiagThreads * m, t = id / (N / 8), c8 = id % (N / 8);
            if (id < S::BCT) st16(Bs + t * NS + 8 * c8, t < len ? rb[m] : uint4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int m = 0; m < XI; ++m) {
            const int id = tid + kSegDiagThreads * m, t = id / (P / 8), c8 = id % (P / 8);
            if (id < S::XT) st16(Xs + t * XS + 8 * c8, t < len ? rx[m] : uint4{0u, 0u, 0u, 0u});
        }
        // (DT) the step sizes of this thread's tokens, from the lanes that formed them
        float dt_i[DT ? TP : 1];
        if (DT) {
            const float delta = softplus_hw(la[0] + dtb);  // of token `lane`
#pragma unroll
            for (int i = 0; i < TP; ++i) dt_i[i] = __shfl(delta, part * TP + i, kWave);
        }
        // log a of this thread's tokens in log2 units, summed down its part of column n
        float cum[TP], run = 0.f;
#pragma unroll
        for (int i = 0; i < TP; ++i) {
            const float l2 = DT ? dt_i[i] * an : la[i] * kLog2eD;
            run += part * TP + i < len ? l2 : 0.f;
            cum[i] = run;
        }
        tot[part * N + n] = run;
        if (c > c0) load_chunk(c - 1);
        __syncthreads();  // staged; partial sums in
        float before = 0.f, last = 0.f;
#pragma unroll
        for (int q = 0; q < S::PARTS; ++q) {
            const float v = tot[q * N + n];
            before += q < part ? v : 0.f;
            last += v;
        }
        // B o W of this thread's tokens in row n (with the front-end's input scale: Delta_t B_tn)
#pragma unroll
        for (int i = 0; i < TP; ++i) {
            const int t = part * TP + i;
            const float w = dexp2(sfx + (last - (before + cum[i])));
            const float sc = DT && prm.scale_input ? dt_i[i] : 1.f;
            BWs[t * NS + n] = (__bf16)((float)Bs[t * NS + n] * (w * sc));
        }
        __syncthreads();  // B o W in
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wave + kSegDiagWaves * j, nb = tile / PB, pb = tile % PB;
            if (tile < NTILE)
#pragma unroll
                for (int k = 0; k < Q / 32; ++k)
                    hs[j] = mfma_bf16(x_frag<false>(BWs, NS, 16 * nb, k, lane), x_frag<false>(Xs, XS, 16 * pb, k, lane),
                                      hs[j]);
        }
        sfx += last;
        // every read of this chunk's tiles done before the next chunk is staged; and the pass
        // stops together once no row's weights are left
        if (__syncthreads_and(sfx < vanish ? 1 : 0)) break;
    }

    if (part == 0) prm.seg_decay[sidx * N + n] = sfx;
    const int l16 = lane % 16, lg = lane / 16;
    float* fin = prm.seg_state + sidx * N * P;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const int tile = wave + kSegDiagWaves * j, nb = tile / PB, pb = tile % PB;
        if (tile >= NTILE) continue;
        float* dst = fin + (16 * nb + 4 * lg) * P + 16 * pb + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i * P] = hs[j][i];
    }
}

template <typename T, int N, int P>
int launch_diag_t(const ForwardLaunch& fl, hipStream_t stream) {
    static bool attr_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    if (!attr_set[dev]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&walk_diag_kernel<T, N, P>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) != hipSuccess)
            return -1;
        attr_set[dev] = true;
    }
    const int64_t units = fl.batch * fl.nheads;
    const int64_t per_xcd = (units + 7) / 8;
    WalkParams wp{fl.x, fl.log_a, fl.Bm, fl.Cm, fl.D, nullptr, fl.init, fl.y, fl.final_state,
                  fl.batch, fl.seqlen, fl.nheads, fl.ngroups, fl.chunk, fl.nchunks, per_xcd};
    wp.seq_off = fl.seq_off;
    wp.total = fl.total;
    const size_t lds = DiagLayout<T, N, P>(fl.chunk).total;
    int k = fl.first_launch;
    return launch_k(fl, k, walk_diag_kernel<T, N, P>, dim3((unsigned)(8 * per_xcd)), dim3(kThreads), lds, stream, wp)
               ? 0
               : -1;
}

#define SSD_DIAG_SHAPES(X)                                                                         \
    X(__bf16, 32, 32) X(__bf16, 32, 64) X(__bf16, 64, 32) X(__bf16, 64, 64) X(__bf16, 128, 32)      \
    X(__bf16, 128, 64) X(float, 16, 32) X(float, 16, 64) X(float, 32, 32) X(float, 32, 64)           \
    X(float, 64, 32) X(float, 64, 64)

}  // namespace

size_t diag_lds_bytes(int dtype, int N, int P, int chunk) {
    if (chunk > 64 || chunk % 16 != 0) return 0;
#define SSD_DLDS(TT, NN, PP) \
    if ((std::is_same<TT, float>::value ? 0 : 1) == dtype && N == NN && P == PP) return DiagLayout<TT, NN, PP>(chunk).total;
    SSD_DIAG_SHAPES(SSD_DLDS)
#undef SSD_DLDS
    return 0;
}

// Workspace of the pipelined diagonal walk: nothing, or for a segmented walk two fp32 states
// and a log2 decay per state row for every (segment, unit).  Packed variable-length batches are
// never segmented.
struct DiagSegLayout {
    int nseg, seg_chunks;
    size_t state, init, decay, total;
};

DiagSegLayout diag_seg_layout(int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, bool varlen) {
    DiagSegLayout l;
    const int64_t units = batch * nheads, nchunks = (seqlen + kDiagQ - 1) / kDiagQ;
    // one round of walk workgroups (one per CU).  Two rounds of half as long segments give the
    // state-only pass (three per CU) more workgroups, but measured slower overall: at the
    // multiscale shape 122 against 125 us per forward (walk 83 against 87 us, state pass 30
    // against 27 us, prefix 4.4 against 5.0 us)
    if (varlen) {
        l.nseg = 1;
        l.seg_chunks = (int)(nchunks > 0 ? nchunks : 1);
    } else {
        l.nseg = walk_segments(units, nchunks, 256, &l.seg_chunks);
    }
    l.state = l.init = l.decay = l.total = 0;
    if (l.nseg > 1) {
        const size_t st = (size_t)l.nseg * units * N * P * 4;
        l.state = 0;
        l.init = st;
        l.decay = 2 * st;
        l.total = 2 * st + ((size_t)l.nseg * units * N * 4 + 255) / 256 * 256;
    }
    return l;
}

bool diag_pipe_shape(int dtype, int N, int P, int chunk) {
    return dtype == 1 && chunk == kDiagQ && (N == 32 || N == 64) && (P == 32 || P == 64);
}

template <int N, int P, bool DT>
int launch_diag_pipe_t(const ForwardLaunch& fl, hipStream_t stream) {
    static bool attr_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    if (!attr_set[dev]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&walk_diag_pipe_kernel<N, P, DT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) != hipSuccess)
            return -1;
        attr_set[dev] = true;
    }
    const DiagSegLayout sl = diag_seg_layout(fl.batch, fl.nheads, fl.seqlen, N, P, fl.seq_off != nullptr);
    const int64_t units = fl.batch * fl.nheads;
    const int64_t per_xcd = (sl.nseg * units + 7) / 8;
    char* ws = reinterpret_cast<char*>(fl.scores);
    WalkParams wp{fl.x, fl.log_a, fl.Bm, fl.Cm, fl.D, nullptr, fl.init, fl.y, fl.final_state,
                  fl.batch, fl.seqlen, fl.nheads, fl.ngroups, fl.chunk, fl.nchunks, per_xcd,
                  sl.seg_chunks, sl.nseg,
                  sl.nseg > 1 ? reinterpret_cast<float*>(ws + sl.init) : nullptr,
                  sl.nseg > 1 ? reinterpret_cast<float*>(ws + sl.state) : nullptr,
                  sl.nseg > 1 ? reinterpret_cast<float*>(ws + sl.decay) : nullptr,
                  fl.dt, fl.dt_bias, fl.A_log, fl.scale_input, fl.seq_off, fl.total};
    const size_t lds = DiagPipeLayout<N, P>::total, slds = SegDiagShape<N, P>::lds_bytes;
    int k = fl.first_launch;
    // (up to kDiagChainMax segments each walk workgroup chains the segment states into its own
    // start state; more take a prefix launch, whose chained states the walk then reads)
    const bool chain = sl.nseg <= kDiagChainMax;
    if (chain) wp.seg_init = nullptr;
    if (sl.nseg > 1) {
        // (the last segment's local state is never needed: only segments 0 .. nseg-2)
        WalkParams sp = wp;
        sp.per_xcd = ((sl.nseg - 1) * units + 7) / 8;
        sp.nseg = sl.nseg - 1;
        if (!launch_k(fl, k, seg_state_diag_kernel<N, P, DT>, dim3((unsigned)(8 * sp.per_xcd)), dim3(kSegDiagThreads),
                      slds, stream, sp))
            return -1;
        if (!chain && launch_seg_prefix(fl, k, fl.init, wp.seg_init, wp.seg_state, wp.seg_decay, units, N, P,
                                        sl.nseg, 1, stream) != 0)
            return -1;
    }
    return launch_k(fl, k, walk_diag_pipe_kernel<N, P, DT>, dim3((unsigned)(8 * per_xcd)), dim3(kDiagThreads), lds,
                    stream, wp)
               ? 0
               : -1;
}

bool diag_pipe_applies(int dtype, int N, int P, int chunk) { return diag_pipe_shape(dtype, N, P, chunk); }

size_t diag_workspace_bytes(int dtype, int64_t batch, int64_t nheads, int64_t seqlen, int N, int P, int chunk,
                            bool varlen) {
    if (!diag_pipe_shape(dtype, N, P, chunk)) return 0;
    return diag_seg_layout(batch, nheads, seqlen, N, P, varlen).total;
}

int launch_forward_diag(const ForwardLaunch& fl, hipStream_t stream) {
    if (diag_pipe_shape(fl.dtype, (int)fl.dstate, (int)fl.headdim, fl.chunk)) {
        const bool dt = fl.dt != nullptr;
        if (fl.dstate == 64 && fl.headdim == 64)
            return dt ? launch_diag_pipe_t<64, 64, true>(fl, stream) : launch_diag_pipe_t<64, 64, false>(fl, stream);
        if (fl.dstate == 64 && fl.headdim == 32)
            return dt ? launch_diag_pipe_t<64, 32, true>(fl, stream) : launch_diag_pipe_t<64, 32, false>(fl, stream);
        if (fl.dstate == 32 && fl.headdim == 64)
            return dt ? launch_diag_pipe_t<32, 64, true>(fl, stream) : launch_diag_pipe_t<32, 64, false>(fl, stream);
        if (fl.dstate == 32 && fl.headdim == 32)
            return dt ? launch_diag_pipe_t<32, 32, true>(fl, stream) : launch_diag_pipe_t<32, 32, false>(fl, stream);
    }
#define SSD_DLAUNCH(TT, NN, PP) \
    if ((std::is_same<TT, float>::value ? 0 : 1) == fl.dtype && fl.dstate == NN && fl.headdim == PP) \
        return launch_diag_t<TT, NN, PP>(fl, stream);
    SSD_DIAG_SHAPES(SSD_DLAUNCH)
#undef SSD_DLAUNCH
    return -2;
}

}  // namespace ssd
