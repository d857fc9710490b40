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
    size_t xt, bt, ht, cc, cf, bu, cum, beta, el, sl, total;
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
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
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

    for (int c = 0; c < prm.nchunks; ++c) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, Tn - t0);
        __syncthreads();  // previous chunk done with every LDS buffer

        // ---- 1. log a into LDS, then running sums down each state column (past the end: 0)
        for (int i = tid; i < QK * N; i += kThreads) {
            const int t = i / N, n = i % N;
            cum[i] = t < len ? (CT)prm.log_a[((b * Tn + t0 + t) * H + h) * N + n] : (CT)0;
        }
        __syncthreads();
        for (int n = tid; n < N; n += kThreads) {
            CT run = 0;
            for (int t = 0; t < QK; ++t) {
                run += cum[t * N + n];
                cum[t * N + n] = run;
            }
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
            const uint4 cv = ok ? ld16(Cg + ((b * Tn + t0 + t) * G + g) * N + cc * VE) : zero;
            const uint4 bv = ok ? ld16(Bg + ((b * Tn + t0 + t) * G + g) * N + cc * VE) : zero;
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
        }
        // x^T and (w o B)^T, four tokens per thread and 16-byte global loads
        for (int item = tid; item < (QK / 4) * (P / VE); item += kThreads) {
            const int rg = item / (P / VE), cc = item % (P / VE);
            uint4 u[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int r = 4 * rg + k;
                u[k] = r < len ? ld16(xg + ((b * Tn + t0 + r) * H + h) * P + cc * VE) : zero;
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
                u[k] = r < len ? ld16(Bg + ((b * Tn + t0 + r) * G + g) * N + cc * VE) : zero;
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
        const int ntiles = nt * (nt + 1) / 2;
        for (int idx = wave; idx < ntiles; idx += kWaves) {
            int tb = 0;
            while (tile_index(tb + 1, 0) <= idx) ++tb;
            const int sb = idx - tile_index(tb, 0);
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
                for (int n = 0; n < N; ++n) {
                    const CT ct = cum[t * N + n];
                    const float craw = (float)Cg[((b * Tn + t0 + min(t, len - 1)) * G + g) * N + n] * (t < len ? 1.f : 0.f);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = 16 * sb + 4 * lg + i;
                        const bool causal = s <= t && s < len;
                        const float braw = causal ? (float)Bg[((b * Tn + t0 + s) * G + g) * N + n] : 0.f;
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
            const int64_t trow = b * Tn + t0 + tl;
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
    const size_t lds = DiagLayout<T, N, P>(fl.chunk).total;
    if (!record_event(fl, 0, stream)) return -1;
    hipLaunchKernelGGL((walk_diag_kernel<T, N, P>), dim3((unsigned)(8 * per_xcd)), dim3(kThreads), lds, stream, wp);
    if (hipGetLastError() != hipSuccess) return -1;
    if (!record_event(fl, 1, stream)) return -1;
    if (fl.n_launches) *fl.n_launches = 1;
    return 0;
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

int launch_forward_diag(const ForwardLaunch& fl, hipStream_t stream) {
#define SSD_DLAUNCH(TT, NN, PP) \
    if ((std::is_same<TT, float>::value ? 0 : 1) == fl.dtype && fl.dstate == NN && fl.headdim == PP) \
        return launch_diag_t<TT, NN, PP>(fl, stream);
    SSD_DIAG_SHAPES(SSD_DLAUNCH)
#undef SSD_DLAUNCH
    return -2;
}

}  // namespace ssd
