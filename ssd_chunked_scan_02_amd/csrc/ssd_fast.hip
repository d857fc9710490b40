// Pipelined chunk walk for bf16 inputs, scalar decay, head dim 64 (the Mamba-2 layer
// shape), gfx950.  Same operator as walk_kernel in ssd_kernels.hip (aiwiki "State Space
// Duality", "Two algorithms for one operator"; llms.blog "The Chunk-Wise SSD Algorithm"),
// organised for latency hiding:
//
//   prep_kernel   per (batch, group, chunk): the causal score tiles S^T = B C^T as bf16
//                 "pairs" (two 16x16 tiles along s, in the exact lane order the walk reads
//                 them as an MFMA operand), and B^T with the token axis permuted the same
//                 way, so every operand the walk reads from global memory is one 16-byte
//                 load per lane.
//   walk2_kernel  one workgroup per (batch, head) walks the chunks; while chunk c is being
//                 computed, every global load chunk c+1 needs (log a, x, C rows, score
//                 pairs, B^T rows) is already in flight into a second register set.  x is
//                 staged row-major in LDS and read as MFMA operands that contract over
//                 tokens with the gfx950 transposing LDS read (ds_read_b64_tr_b16): a
//                 16-lane group whose lane 4j+q points at row r_j, columns 4q..4q+3 returns
//                 in lane i column i of rows r_0..r_3.  One workgroup barrier per chunk.
//
// K order inside a 32-token MFMA step: lane group g, element j holds token
//   kperm(g, j) = 4g + j (j < 4),  16 + 4g + (j - 4) (j >= 4)
// which is the row set an accumulator lane of two stacked 16x16 tiles owns, so the masked
// scores enter the intra-chunk product straight from registers.

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kP = 64;            // head dim handled here
constexpr int kXStr = kP + 8;     // LDS row stride of the x tile, elements

__host__ __device__ constexpr int pair_base(int tb) {
    return (tb % 2 == 0) ? (tb / 2) * (tb / 2 + 1) : (tb / 2 + 1) * (tb / 2 + 1);
}
__host__ __device__ constexpr int n_pairs(int nt) { return pair_base(nt); }
__device__ __forceinline__ int kperm(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

__device__ __forceinline__ v4i16 lds_read_tr(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

// x fragment for K step k and p block pb, tokens in kperm order: lane (g, i) receives
// x[32k + kperm(g, j)][16 pb + i], j = 0..7.
__device__ __forceinline__ bf16x8 x_frag(const __bf16* xs, int pb, int k, int lane) {
    const int g = lane / 16, jr = (lane % 16) / 4, q = lane % 4;
    const __bf16* base = xs + (32 * k + 4 * g + jr) * kXStr + 16 * pb + 4 * q;
    const v4i16 lo = lds_read_tr(base);
    const v4i16 hi = lds_read_tr(base + 16 * kXStr);
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------------------
template <int N, int Q>
__global__ void __launch_bounds__(kThreads) prep_kernel(PrepParams prm) {
    constexpr int NT = Q / 16;
    constexpr int NPAIR = n_pairs(NT);
    constexpr int NS = N + 8;
    __shared__ __align__(16) __bf16 Bs[Q * NS];
    __shared__ __align__(16) __bf16 Cs[Q * NS];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int l16 = lane % 16, lg = lane / 16;
    const int64_t blk = blockIdx.x;
    const int c = (int)(blk % prm.nchunks);
    const int64_t bg = blk / prm.nchunks;
    const int64_t b = bg / prm.ngroups, g = bg % prm.ngroups;
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, prm.seqlen - t0);
    const __bf16* Bg = static_cast<const __bf16*>(prm.Bm);
    const __bf16* Cg = static_cast<const __bf16*>(prm.Cm);
    const uint4 zero = {0u, 0u, 0u, 0u};

    for (int id = tid; id < Q * (N / 8); id += kThreads) {
        const int row = id / (N / 8), c8 = id % (N / 8);
        const int64_t off = ((b * prm.seqlen + t0 + row) * prm.ngroups + g) * N + 8 * c8;
        st16(Bs + row * NS + 8 * c8, row < len ? ld16(Bg + off) : zero);
        st16(Cs + row * NS + 8 * c8, row < len ? ld16(Cg + off) : zero);
    }
    __syncthreads();

    // B^T with tokens in kperm order: bt[n][32k + 8g + j] = B[32k + kperm(g, j)][n]
    __bf16* bt = prm.bt + blk * (int64_t)N * Q;
    for (int id = tid; id < N * (Q / 8); id += kThreads) {
        const int n = id / (Q / 8), q8 = id % (Q / 8);
        const int k = q8 / 4, gg = q8 % 4;
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = Bs[(32 * k + kperm(gg, j)) * NS + n];
        *reinterpret_cast<bf16x8*>(bt + n * Q + 8 * q8) = v;
    }

    // score pairs: pair (tb, k) = tiles S^T[s block 2k][tb] and S^T[s block 2k+1][tb]
    __bf16* pairs = prm.pairs + blk * (int64_t)NPAIR * 512;
    for (int tb = 0; tb < NT; ++tb) {
        for (int k = 0; 2 * k <= tb; ++k) {
            const int idx = pair_base(tb) + k;
            if (idx % kWaves != wave) continue;
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int sb = 2 * k + h;
                if (sb > tb) continue;
#pragma unroll
                for (int kk = 0; kk < N / 32; ++kk) {
                    const bf16x8 a = as_bf16x8(ld16(Bs + (16 * sb + l16) * NS + 32 * kk + 8 * lg));
                    const bf16x8 bb = as_bf16x8(ld16(Cs + (16 * tb + l16) * NS + 32 * kk + 8 * lg));
                    acc[h] = mfma_bf16(a, bb, acc[h]);
                }
            }
            const bf16x8 v = {(__bf16)acc[0][0], (__bf16)acc[0][1], (__bf16)acc[0][2], (__bf16)acc[0][3],
                              (__bf16)acc[1][0], (__bf16)acc[1][1], (__bf16)acc[1][2], (__bf16)acc[1][3]};
            *reinterpret_cast<bf16x8*>(pairs + idx * 512 + lane * 8) = v;
        }
    }
}

// ---------------------------------------------------------------------------------------
template <int N, int Q>
struct Prefetch {
    static constexpr int NT = Q / 16, TBW = NT / 4, KS = Q / 32, KN = N / 32, NBW = N / 64;
    static constexpr int LA = Q / 64, XCH = Q * 8 / kThreads;
    float la[LA];
    uint4 xs[XCH];
    uint4 cf[TBW][KN];
    uint4 sp[TBW][KS];
    uint4 bt[NBW][KS];
};

// 16-token block handled by wave `wave` in its r-th round (snake order balances the causal
// work across the four waves).
__device__ __forceinline__ int wave_tb(int r, int wave) { return (r % 2 == 0) ? 4 * r + wave : 4 * r + 3 - wave; }

template <int N, int Q>
__global__ void __launch_bounds__(kThreads) walk2_kernel(Walk2Params prm) {
    using PF = Prefetch<N, Q>;
    constexpr int TBW = PF::TBW, KS = PF::KS, KN = PF::KN, NBW = PF::NBW, LA = PF::LA, XCH = PF::XCH;
    constexpr int NT = PF::NT, NPAIR = n_pairs(NT), PB = kP / 16, HS = N + 8;

    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, prm.batch * H);
    if (unit < 0) return;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int l16 = lane % 16, lg = lane / 16;
    const int nchunks = prm.nchunks;

    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Xs = reinterpret_cast<__bf16*>(smem);             // [2][Q][kXStr]
    __bf16* Hs = Xs + 2 * Q * kXStr;                           // [2][kP][HS]  H^T, bf16
    float* wa = reinterpret_cast<float*>(Hs + 2 * kP * HS) + wave * 3 * Q;  // this wave's
    float* cum_s = wa;                                         // running sums of log a
    float* ecum_s = wa + Q;                                    // exp(cum_t)
    float* wdec_s = wa + 2 * Q;                                // exp(cum_last - cum_s)

    const __bf16* xg = static_cast<const __bf16*>(prm.x);
    const __bf16* Cg = static_cast<const __bf16*>(prm.Cm);
    __bf16* yg = static_cast<__bf16*>(prm.y);
    const uint4 zero = {0u, 0u, 0u, 0u};
    const float dskip = prm.D ? prm.D[h] : 0.f;
    const bool has_skip = prm.D != nullptr;

    auto issue = [&](int c, PF& p) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, Tn - t0);
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const int tok = lane * LA + j;
            p.la[j] = tok < len ? prm.log_a[(b * Tn + t0 + tok) * H + h] : 0.f;
        }
#pragma unroll
        for (int m = 0; m < XCH; ++m) {
            const int id = tid + kThreads * m, row = id / 8, c16 = id % 8;
            p.xs[m] = row < len ? ld16(xg + ((b * Tn + t0 + row) * H + h) * kP + 8 * c16) : zero;
        }
#pragma unroll
        for (int r = 0; r < TBW; ++r) {
            const int t = 16 * wave_tb(r, wave) + l16;
            const __bf16* crow = Cg + ((b * Tn + t0 + t) * G + g) * N + 8 * lg;
#pragma unroll
            for (int k = 0; k < KN; ++k) p.cf[r][k] = t < len ? ld16(crow + 32 * k) : zero;
        }
        const int64_t cblk = (b * G + g) * nchunks + c;
        const __bf16* pairs = prm.pairs + cblk * NPAIR * 512 + lane * 8;
#pragma unroll
        for (int r = 0; r < TBW; ++r) {
            const int tb = wave_tb(r, wave);
#pragma unroll
            for (int k = 0; k < KS; ++k) p.sp[r][k] = (2 * k <= tb) ? ld16(pairs + (pair_base(tb) + k) * 512) : zero;
        }
        const __bf16* bt = prm.bt + cblk * N * Q + 8 * lg;
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn) {
            const int n = 16 * (wave + 4 * jn) + l16;
#pragma unroll
            for (int k = 0; k < KS; ++k) p.bt[jn][k] = ld16(bt + n * Q + 32 * k);
        }
    };

    // ---- state (fp32): tiles (nb = wave + 4 jn, pb), accumulator layout
    f32x4 hs[NBW][PB];
#pragma unroll
    for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            hs[jn][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (prm.init) {
                const int n = 16 * (wave + 4 * jn) + 4 * lg;
                const float* src = prm.init + (unit * N + n) * kP + 16 * pb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) hs[jn][pb][i] = src[i * kP];
            }
        }
    auto write_state = [&](__bf16* hsm) {
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int n = 16 * (wave + 4 * jn) + 4 * lg;
                store4(hsm + (16 * pb + l16) * HS + n, hs[jn][pb][0], hs[jn][pb][1], hs[jn][pb][2], hs[jn][pb][3]);
            }
    };
    write_state(Hs);

    auto body = [&](int c, PF& cur, PF& nxt) {
        const int64_t t0 = (int64_t)c * Q;
        const int len = (int)min((int64_t)Q, Tn - t0);
        __bf16* xs = Xs + (c & 1) * Q * kXStr;
        const __bf16* hcur = Hs + (c & 1) * kP * HS;
        __bf16* hnext = Hs + ((c + 1) & 1) * kP * HS;

        // 1. running sums of log a over the chunk, computed by every wave for itself
        float v[LA];
        float run = 0.f;
#pragma unroll
        for (int j = 0; j < LA; ++j) { run += cur.la[j]; v[j] = run; }
        float incl = run;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float o = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += o;
        }
        const float excl = incl - run;
        const float cum_last = __shfl(incl, kWave - 1, kWave);
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const float cv = excl + v[j];
            const int tok = lane * LA + j;
            cum_s[tok] = cv;
            ecum_s[tok] = __expf(cv);
            wdec_s[tok] = __expf(cum_last - cv);
        }
        // 2. x of this chunk into LDS, row-major
#pragma unroll
        for (int m = 0; m < XCH; ++m) {
            const int id = tid + kThreads * m, row = id / 8, c16 = id % 8;
            st16(xs + row * kXStr + 8 * c16, cur.xs[m]);
        }
        __syncthreads();
        // 3. next chunk's loads go out now and land while this chunk computes
        if (c + 1 < nchunks) issue(c + 1, nxt);

        // 4. outputs of this wave's 16-token blocks
        bf16x8 hf[PB][KN];
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int k = 0; k < KN; ++k) hf[pb][k] = as_bf16x8(ld16(hcur + (16 * pb + l16) * HS + 32 * k + 8 * lg));
#pragma unroll
        for (int r = 0; r < TBW; ++r) {
            const int tb = wave_tb(r, wave);
            const int t = 16 * tb + l16;
            f32x4 acc[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
            // carried state: C_t H_{k-1}, times exp(cum_t)
#pragma unroll
            for (int k = 0; k < KN; ++k) {
                const bf16x8 cb = as_bf16x8(cur.cf[r][k]);
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) acc[pb] = mfma_bf16(hf[pb][k], cb, acc[pb]);
            }
            const float ec = ecum_s[t];
            const float cum_t = cum_s[t];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[pb] *= ec;
            // inside the chunk: (S o L) X, the mask selected before the exp
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                if (2 * k > tb) continue;
                const bf16x8 s8 = as_bf16x8(cur.sp[r][k]);
                const f32x4 ca = *reinterpret_cast<const f32x4*>(cum_s + 32 * k + 4 * lg);
                const f32x4 cbv = *reinterpret_cast<const f32x4*>(cum_s + 32 * k + 16 + 4 * lg);
                bf16x8 bop;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = 32 * k + kperm(lg, j);
                    const float cs = j < 4 ? ca[j] : cbv[j - 4];
                    const bool causal = s <= t;
                    const float d = causal ? cum_t - cs : 0.f;
                    bop[j] = (__bf16)(causal ? (float)s8[j] * __expf(d) : 0.f);
                }
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) acc[pb] = mfma_bf16(x_frag(xs, pb, k, lane), bop, acc[pb]);
            }
            if (has_skip) {
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(xs + t * kXStr + 16 * pb + 4 * lg);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[pb][i] += dskip * (float)x4[i];
                }
            }
            if (t < len) {
                __bf16* yr = yg + ((b * Tn + t0 + t) * H + h) * kP + 4 * lg;
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) store4(yr + 16 * pb, acc[pb][0], acc[pb][1], acc[pb][2], acc[pb][3]);
            }
        }

        // 5. state: H_k = exp(cum_last) H_{k-1} + (w o B)^T X
        const float el = __expf(cum_last);
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) hs[jn][pb] *= el;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(wdec_s + 32 * k + 4 * lg);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(wdec_s + 32 * k + 16 + 4 * lg);
            bf16x8 a[NBW];
#pragma unroll
            for (int jn = 0; jn < NBW; ++jn) {
                const bf16x8 raw = as_bf16x8(cur.bt[jn][k]);
#pragma unroll
                for (int j = 0; j < 8; ++j) a[jn][j] = (__bf16)((float)raw[j] * (j < 4 ? w0[j] : w1[j - 4]));
            }
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const bf16x8 xf = x_frag(xs, pb, k, lane);
#pragma unroll
                for (int jn = 0; jn < NBW; ++jn) hs[jn][pb] = mfma_bf16(a[jn], xf, hs[jn][pb]);
            }
        }
        write_state(hnext);
    };

    PF pa, pb_;
    issue(0, pa);
    for (int c = 0; c < nchunks; c += 2) {
        body(c, pa, pb_);
        if (c + 1 < nchunks) body(c + 1, pb_, pa);
    }

    if (prm.final_state) {
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int n = 16 * (wave + 4 * jn) + 4 * lg;
                float* dst = prm.final_state + (unit * N + n) * kP + 16 * pb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * kP] = hs[jn][pb][i];
            }
    }
}

template <int N, int Q>
size_t walk2_lds() {
    return (size_t)(2 * Q * kXStr + 2 * kP * (N + 8)) * 2 + (size_t)kWaves * 3 * Q * 4;
}

template <int N, int Q>
int launch_fast_t(const ForwardLaunch& fl, hipStream_t stream) {
    constexpr int NPAIR = n_pairs(Q / 16);
    __bf16* pairs = reinterpret_cast<__bf16*>(fl.scores);
    const int64_t nblk = fl.batch * fl.ngroups * fl.nchunks;
    __bf16* bt = pairs + nblk * NPAIR * 512;
    PrepParams pp{fl.Bm, fl.Cm, pairs, bt, fl.seqlen, fl.ngroups, fl.nchunks};
    if (!record_event(fl, 0, stream)) return -1;
    hipLaunchKernelGGL((prep_kernel<N, Q>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, pp);
    if (hipGetLastError() != hipSuccess) return -1;

    const int64_t units = fl.batch * fl.nheads;
    const int64_t per_xcd = (units + 7) / 8;
    Walk2Params wp{fl.x, fl.log_a, fl.Cm, fl.D, pairs, bt, fl.init, fl.y, fl.final_state,
                   fl.batch, fl.seqlen, fl.nheads, fl.ngroups, fl.nchunks, per_xcd};
    static bool attr_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    if (!attr_set[dev]) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&walk2_kernel<N, Q>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) != hipSuccess)
            return -1;
        attr_set[dev] = true;
    }
    if (!record_event(fl, 1, stream)) return -1;
    const size_t lds = walk2_lds<N, Q>();
    hipLaunchKernelGGL((walk2_kernel<N, Q>), dim3((unsigned)(8 * per_xcd)), dim3(kThreads), lds, stream, wp);
    if (hipGetLastError() != hipSuccess) return -1;
    if (!record_event(fl, 2, stream)) return -1;
    if (fl.n_launches) *fl.n_launches = 2;
    return 0;
}

}  // namespace

bool fast_path_applies(int dtype, int decay, int N, int P, int chunk) {
    return dtype == 1 && decay == 0 && P == kP && (N == 64 || N == 128) && (chunk == 64 || chunk == 128);
}

size_t fast_workspace_bytes(int64_t batch, int64_t ngroups, int64_t nchunks, int N, int chunk) {
    const int64_t nblk = batch * ngroups * nchunks;
    return (size_t)nblk * ((size_t)n_pairs(chunk / 16) * 1024 + (size_t)N * chunk * 2);
}

int launch_forward_fast(const ForwardLaunch& fl, hipStream_t stream) {
    const int N = (int)fl.dstate, Q = fl.chunk;
    if (N == 64 && Q == 64) return launch_fast_t<64, 64>(fl, stream);
    if (N == 64 && Q == 128) return launch_fast_t<64, 128>(fl, stream);
    if (N == 128 && Q == 64) return launch_fast_t<128, 64>(fl, stream);
    if (N == 128 && Q == 128) return launch_fast_t<128, 128>(fl, stream);
    return -2;
}

}  // namespace ssd
