// Pipelined chunk walk for bf16 inputs, scalar decay, head dim 64 (the Mamba-2 layer
// shape), gfx950.  Same operator as walk_kernel in ssd_kernels.hip (aiwiki "State Space
// Duality", "Two algorithms for one operator"; llms.blog "The Chunk-Wise SSD Algorithm"),
// organised for latency hiding and a small VALU budget:
//
//   prep_kernel   per (batch, group, chunk): the causal score tiles S^T = B C^T as bf16
//                 "pairs" (two 16x16 tiles along s) and the B^T MFMA operand fragments, both
//                 stored in the lane order the walk reads them, so each is one coalesced
//                 16-byte load per lane.
//   walk5_kernel  one workgroup (8 waves, two roles) per (batch, head) walks the chunks with
//                 the fp32 N x P state in registers.  Every global operand of chunk c+1 is
//                 loaded into registers right after its last use in chunk c (one register
//                 set, rolling), and the one workgroup barrier per chunk orders LDS only, so
//                 those loads stay in flight across it.  x is staged row-major in LDS and read as MFMA operands
//                 that contract over tokens with the transposing LDS read ds_read_b64_tr_b16
//                 (a 16-lane group whose lane 4j+q points at row r_j, columns 4q..4q+3 returns
//                 in lane i column i of rows r_0..r_3).
//
// Token order inside a 32-token MFMA step: lane group g, element j holds token
//   kperm(g, j) = 4g + j (j < 4),  16 + 4g + (j - 4) (j >= 4),
// the row set an accumulator lane of two stacked 16x16 tiles owns, so masked scores feed the
// intra-chunk product straight from registers.
//
// Decay mask without an exp per score: for a 16-token output block tb starting at token a
// and any token s before that block, exp(cum_t - cum_s) = f_t * beta(tb, sb) * u_s with
//   f_t = exp(cum_t - cum_a),  beta(tb, sb) = exp(cum_a - cum_e),  u_s = exp(cum_e - cum_s),
// e the last token of s's 16-token block; each factor is exp of a non-positive number.  Only
// the scores of the 32-token step that contains the diagonal block take exact exps.

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kP = 64;            // head dim handled here
constexpr int kXStr = kP + 8;     // LDS row stride of the x tile, elements
constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate with lgkmcnt = 0 and the vector-memory and export counters left at
// their maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitLgkm0 = 0xC07F;

__host__ __device__ constexpr int pair_base(int tb) {
    return (tb % 2 == 0) ? (tb / 2) * (tb / 2 + 1) : (tb / 2 + 1) * (tb / 2 + 1);
}
__host__ __device__ constexpr int n_pairs(int nt) { return pair_base(nt); }
__device__ __forceinline__ int kperm(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

__device__ __forceinline__ v4i16 lds_read_tr(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

// Barrier that orders LDS accesses only: global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Operand fragment of a row-major [token][col] bf16 tile in LDS, contracting over tokens:
// lane (g, i) receives tile[32k + kperm(g, j)][col0 + i], j = 0..7.
__device__ __forceinline__ bf16x8 token_frag(const __bf16* tile, int stride, int col0, int k, int lane) {
    const int g = lane / 16, jr = (lane % 16) / 4, q = lane % 4;
    const __bf16* base = tile + (32 * k + 4 * g + jr) * stride + col0 + 4 * q;
    const v4i16 lo = lds_read_tr(base);
    const v4i16 hi = lds_read_tr(base + 16 * stride);
    const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// 2^x on the hardware unit (v_exp_f32); results below the normal range are not kept, which
// only affects decay factors under 2^-126.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16x8 -> 8 floats (exact widening).
__device__ __forceinline__ void unpack8(bf16x8 v, float (&f)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (float)v[j];
}

// ---------------------------------------------------------------------------------------
// prep_kernel: kPrepParts workgroups per (batch, group, chunk); each stages the chunk's B and
// C rows in LDS and writes its share of
//   pairs[(b,g,c)][pair(tb,k)][lane][8]: S^T[32k + kperm(lg, j)][16 tb + l16] (0 where the
//       second tile lies above the diagonal), pair(tb,k) = pair_base(tb) + k, 2k <= tb;
//   btf[(b,g,c)][nb][k][lane][8]: B[32k + kperm(lg, j)][16 nb + l16]  (the B^T operand).
constexpr int kPrepParts = 4;

template <int N, int Q>
__global__ void __launch_bounds__(kThreads) prep_kernel(PrepParams prm) {
    constexpr int NT = Q / 16, KS = Q / 32, NB = N / 16;
    constexpr int NPAIR = n_pairs(NT);
    constexpr int NS = N + 8;
    constexpr int WORKERS = kPrepParts * kWaves;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Bs = reinterpret_cast<__bf16*>(smem);   // [Q][NS]
    __bf16* Cs = Bs + Q * NS;                       // [Q][NS]
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int l16 = lane % 16, lg = lane / 16;
    const int part = blockIdx.x % kPrepParts;
    const int64_t blk = blockIdx.x / kPrepParts;
    const int worker = part * kWaves + wave;
    const int c = (int)(blk % prm.nchunks);
    const int64_t bg = blk / prm.nchunks;
    const int64_t b = bg / prm.ngroups, g = bg % prm.ngroups;
    const int64_t t0 = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, prm.seqlen - t0);
    const __bf16* Bg = static_cast<const __bf16*>(prm.Bm);
    const __bf16* Cg = static_cast<const __bf16*>(prm.Cm);
    const uint4 zero = {0u, 0u, 0u, 0u};

    constexpr int ITEMS = Q * (N / 8) / kThreads;
    uint4 vb[ITEMS], vc[ITEMS];
#pragma unroll
    for (int m = 0; m < ITEMS; ++m) {
        const int id = tid + kThreads * m, row = id / (N / 8), c8 = id % (N / 8);
        const int64_t off = ((b * prm.seqlen + t0 + min(row, len - 1)) * prm.ngroups + g) * N + 8 * c8;
        vb[m] = ld16(Bg + off);
        vc[m] = ld16(Cg + off);
    }
#pragma unroll
    for (int m = 0; m < ITEMS; ++m) {
        const int id = tid + kThreads * m, row = id / (N / 8), c8 = id % (N / 8);
        st16(Bs + row * NS + 8 * c8, row < len ? vb[m] : zero);
        st16(Cs + row * NS + 8 * c8, row < len ? vc[m] : zero);
    }
    __syncthreads();

    __bf16* btf = prm.bt + blk * (int64_t)NB * KS * 512 + lane * 8;
    for (int f = worker; f < NB * KS; f += WORKERS) {
        const int nb = f / KS, k = f % KS;
        *reinterpret_cast<bf16x8*>(btf + f * 512) = token_frag(Bs, NS, 16 * nb, k, lane);
    }

    __bf16* pairs = prm.pairs + blk * (int64_t)NPAIR * 512 + lane * 8;
    for (int idx = worker; idx < NPAIR; idx += WORKERS) {
        int tb = 0;
        while (pair_base(tb + 1) <= idx) ++tb;
        const int k = idx - pair_base(tb);
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int sb = 2 * k + hh;
            if (sb > tb) continue;
#pragma unroll
            for (int kk = 0; kk < N / 32; ++kk) {
                const bf16x8 a = as_bf16x8(ld16(Bs + (16 * sb + l16) * NS + 32 * kk + 8 * lg));
                const bf16x8 bb = as_bf16x8(ld16(Cs + (16 * tb + l16) * NS + 32 * kk + 8 * lg));
                acc[hh] = mfma_bf16(a, bb, acc[hh]);
            }
        }
        const bf16x8 v = {(__bf16)acc[0][0], (__bf16)acc[0][1], (__bf16)acc[0][2], (__bf16)acc[0][3],
                          (__bf16)acc[1][0], (__bf16)acc[1][1], (__bf16)acc[1][2], (__bf16)acc[1][3]};
        *reinterpret_cast<bf16x8*>(pairs + idx * 512) = v;
    }
}

// ---------------------------------------------------------------------------------------
// walk5_kernel: 8 waves per (batch, head) in two roles; wave i runs on SIMD i % 4, so each
// SIMD interleaves one wave of each role.
//   output waves 0-3: y of their 16-token blocks for chunk c, from H_{k-1} (LDS), the staged
//       x and decay factors of chunk c, C rows and score pairs (registers).
//   state waves 4-7: H_k = exp(cum_last) H_{k-1} + B^T (w o X) for chunk c, written to the
//       other LDS state buffer; then they prepare chunk c+1 for everyone: running sums of
//       log a (wave-wide DPP scan), decay factors, x staged raw and weighted by w.
// One LDS barrier per chunk; everything written for chunk c+1 goes to the other of two
// buffers, whose previous contents (chunk c-1) every wave finished before the last barrier.
constexpr int kWalkWaves = 8;
constexpr int kWalkThreads = kWalkWaves * kWave;

// 16-token block handled by output wave `ow` in its r-th round (snake order balances the
// causal work across the four output waves).
__device__ __forceinline__ int wave_tb(int r, int ow) { return (r % 2 == 0) ? 4 * r + ow : 4 * r + 3 - ow; }

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and row broadcasts.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_src(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_src<0x111, 0xf>(x);  // row_shr:1
    x += dpp_src<0x112, 0xf>(x);  // row_shr:2
    x += dpp_src<0x114, 0xf>(x);  // row_shr:4
    x += dpp_src<0x118, 0xf>(x);  // row_shr:8
    x += dpp_src<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_src<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

template <int N, int Q>
struct WalkShape {
    static constexpr int NT = Q / 16, TBW = NT / 4, KS = Q / 32, KN = N / 32, NBW = N / 64;
    static constexpr int LA = Q / 64, QW = Q / 4, XCH = QW * 8 / kWave, NPAIR = n_pairs(NT);
    static constexpr int PB = kP / 16, HS = N + 8;
    static constexpr int FSZ = 4 * Q + NT * NT + NT;  // floats of one decay-factor buffer
    static constexpr size_t lds_bytes = (size_t)(4 * Q * kXStr + 2 * kP * HS) * 2 + (size_t)2 * FSZ * 4;
};

template <int N, int Q>
__global__ void __launch_bounds__(kWalkThreads) walk5_kernel(Walk2Params prm) {
    using WS = WalkShape<N, Q>;
    constexpr int NT = WS::NT, TBW = WS::TBW, KS = WS::KS, KN = WS::KN, NBW = WS::NBW;
    constexpr int LA = WS::LA, QW = WS::QW, XCH = WS::XCH, NPAIR = WS::NPAIR, PB = WS::PB, HS = WS::HS;
    constexpr int FSZ = WS::FSZ;

    const int64_t H = prm.nheads, G = prm.ngroups, Tn = prm.seqlen;
    const int64_t unit = xcd_work_index(blockIdx.x, prm.per_xcd, prm.batch * H);
    if (unit < 0) return;
    const int64_t b = unit / H, h = unit % H, g = h / (H / G);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int l16 = lane % 16, lg = lane / 16;
    const int rw = wave % 4;  // index of the wave within its role
    const int nchunks = prm.nchunks;

    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Xs = reinterpret_cast<__bf16*>(smem);             // [2][Q][kXStr] x
    __bf16* Xw = Xs + 2 * Q * kXStr;                           // [2][Q][kXStr] w o x
    __bf16* Hs = Xw + 2 * Q * kXStr;                           // [2][kP][HS] H^T, bf16
    float* Fs = reinterpret_cast<float*>(Hs + 2 * kP * HS);    // [2][FSZ] decay factors
    // one factor buffer: cum2 (log2 e times running sum of log a), u_s, f_t, w_s, beta, exp(cum_a)
    auto fcum2 = [&](int buf) { return Fs + buf * FSZ; };
    auto fu = [&](int buf) { return Fs + buf * FSZ + Q; };
    auto ff = [&](int buf) { return Fs + buf * FSZ + 2 * Q; };
    auto fw = [&](int buf) { return Fs + buf * FSZ + 3 * Q; };
    auto fbeta = [&](int buf) { return Fs + buf * FSZ + 4 * Q; };
    auto fea = [&](int buf) { return Fs + buf * FSZ + 4 * Q + NT * NT; };

    const __bf16* xg = static_cast<const __bf16*>(prm.x);
    const __bf16* Cg = static_cast<const __bf16*>(prm.Cm);
    __bf16* yg = static_cast<__bf16*>(prm.y);
    const uint4 zero = {0u, 0u, 0u, 0u};
    const int64_t cbase = (b * G + g) * (int64_t)nchunks;
    auto chunk_len = [&](int c) { return (int)min((int64_t)Q, Tn - (int64_t)c * Q); };

    if (wave < 4) {
        // ================================ output waves
        const int ow = rw;
        const float dskip = prm.D ? prm.D[h] : 0.f;
        const bool has_skip = prm.D != nullptr;
        // Loads are unconditional with rows clamped into the chunk, so the compiler counts the
        // loads in flight exactly; rows past a short chunk's end are never stored.
        uint4 cf[TBW][KN], sp[TBW][KS];
        auto load_c = [&](int c) {
            const int64_t t0 = (int64_t)c * Q;
            const int last = chunk_len(c) - 1;
#pragma unroll
            for (int r = 0; r < TBW; ++r) {
                const int t = min(16 * wave_tb(r, ow) + l16, last);
                const __bf16* crow = Cg + ((b * Tn + t0 + t) * G + g) * N + 8 * lg;
#pragma unroll
                for (int k = 0; k < KN; ++k) cf[r][k] = ld16(crow + 32 * k);
            }
        };
        auto load_s = [&](int c) {
            const __bf16* pairs = prm.pairs + (cbase + c) * NPAIR * 512 + lane * 8;
#pragma unroll
            for (int r = 0; r < TBW; ++r) {
                const int tb = wave_tb(r, ow);
#pragma unroll
                for (int k = 0; k < KS; ++k) sp[r][k] = ld16(pairs + (pair_base(tb) + min(k, tb / 2)) * 512);
            }
        };
        load_c(0);
        load_s(0);
        int kdmax = 0;
#pragma unroll
        for (int r = 0; r < TBW; ++r) kdmax = max(kdmax, wave_tb(r, ow) / 2);
        lds_barrier();

        for (int c = 0; c < nchunks; ++c) {
            const int64_t t0 = (int64_t)c * Q;
            const int len = chunk_len(c);
            const int cn = min(c + 1, nchunks - 1);
            const int buf = c & 1;
            const __bf16* xsm = Xs + buf * Q * kXStr;
            const __bf16* hcur = Hs + buf * kP * HS;
            const float* cum2 = fcum2(buf);
            const float* uf = fu(buf);
            const float* ffa = ff(buf);
            const float* beta = fbeta(buf);
            const float* ea = fea(buf);

            // carried state: acc = exp(cum_a) C_t H_{k-1}
            f32x4 acc[TBW][PB];
#pragma unroll
            for (int r = 0; r < TBW; ++r)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) acc[r][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KN; ++k)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    const bf16x8 hf = as_bf16x8(ld16(hcur + (16 * pb + l16) * HS + 32 * k + 8 * lg));
#pragma unroll
                    for (int r = 0; r < TBW; ++r) acc[r][pb] = mfma_bf16(hf, as_bf16x8(cf[r][k]), acc[r][pb]);
                }
            load_c(cn);
#pragma unroll
            for (int r = 0; r < TBW; ++r) {
                const float sc = ea[wave_tb(r, ow)];
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) acc[r][pb] *= sc;
            }

            // inside the chunk: (S o L) X over the 32-token steps
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                if (k > kdmax) break;
                bf16x8 xf[PB];
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) xf[pb] = token_frag(xsm, kXStr, 16 * pb, k, lane);
                const f32x4 u0 = *reinterpret_cast<const f32x4*>(uf + 32 * k + 4 * lg);
                const f32x4 u1 = *reinterpret_cast<const f32x4*>(uf + 32 * k + 16 + 4 * lg);
#pragma unroll
                for (int r = 0; r < TBW; ++r) {
                    const int tb = wave_tb(r, ow);
                    const int kd = tb / 2;  // step holding the diagonal block
                    if (k > kd) continue;
                    float s8[8];
                    unpack8(as_bf16x8(sp[r][k]), s8);
                    bf16x8 bop;
                    if (k < kd) {
                        const float b0 = beta[tb * NT + 2 * k], b1 = beta[tb * NT + 2 * k + 1];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            bop[j] = (__bf16)(s8[j] * (b0 * u0[j]));
                            bop[j + 4] = (__bf16)(s8[j + 4] * (b1 * u1[j]));
                        }
                    } else {
                        // remaining factor f_t first, then the exact diagonal step
                        const int t = 16 * tb + l16;
                        const float ft = ffa[t];
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb) acc[r][pb] *= ft;
                        const float ct = cum2[t];
                        const f32x4 c0 = *reinterpret_cast<const f32x4*>(cum2 + 32 * k + 4 * lg);
                        const f32x4 c1 = *reinterpret_cast<const f32x4*>(cum2 + 32 * k + 16 + 4 * lg);
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int s = 32 * k + kperm(lg, j);
                            const float cs = j < 4 ? c0[j] : c1[j - 4];
                            const bool causal = s <= t;
                            bop[j] = (__bf16)(causal ? s8[j] * fexp2(causal ? ct - cs : 0.f) : 0.f);
                        }
                    }
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) acc[r][pb] = mfma_bf16(xf[pb], bop, acc[r][pb]);
                }
            }
            load_s(cn);

            // skip term, outputs
#pragma unroll
            for (int r = 0; r < TBW; ++r) {
                const int t = 16 * wave_tb(r, ow) + l16;
                if (has_skip) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                        const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(xsm + t * kXStr + 16 * pb + 4 * lg);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[r][pb][i] += dskip * (float)x4[i];
                    }
                }
                if (t < len) {
                    __bf16* yr = yg + ((b * Tn + t0 + t) * H + h) * kP + 4 * lg;
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
                        store4(yr + 16 * pb, acc[r][pb][0], acc[r][pb][1], acc[r][pb][2], acc[r][pb][3]);
                }
            }
            lds_barrier();
        }
    } else {
        // ================================ state waves
        const int sw = rw;
        float la[LA];
        uint4 xs[XCH];
        uint4 bt[NBW][KS];
        // log a of the whole chunk (every state wave scans it all) and x rows of this wave's
        // quarter of the chunk; rows clamped into the chunk, masked when staged
        auto load_lax = [&](int c) {
            const int64_t t0 = (int64_t)c * Q;
            const int last = chunk_len(c) - 1;
#pragma unroll
            for (int j = 0; j < LA; ++j) la[j] = prm.log_a[(b * Tn + t0 + min(lane * LA + j, last)) * H + h];
#pragma unroll
            for (int m = 0; m < XCH; ++m) {
                const int id = lane + kWave * m, row = min(QW * sw + id / 8, last), c16 = id % 8;
                xs[m] = ld16(xg + ((b * Tn + t0 + row) * H + h) * kP + 8 * c16);
            }
        };
        auto load_b = [&](int c) {
            const __bf16* btf = prm.bt + (cbase + c) * (N / 16) * KS * 512 + lane * 8;
#pragma unroll
            for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
                for (int k = 0; k < KS; ++k) bt[jn][k] = ld16(btf + ((sw + 4 * jn) * KS + k) * 512);
        };
        // Decay factors of chunk c into factor buffer c & 1 and x of chunk c into the x
        // buffers c & 1.  Returns exp(cum_last).
        auto prepare = [&](int c) -> float {
            const int len = chunk_len(c);
            const int buf = c & 1;
            float cum[LA], run = 0.f;
#pragma unroll
            for (int j = 0; j < LA; ++j) { run += (lane * LA + j < len) ? la[j] : 0.f; cum[j] = run; }
            const float incl = wave_inclusive_sum(run);
            const float excl = incl - run;
#pragma unroll
            for (int j = 0; j < LA; ++j) cum[j] = (excl + cum[j]) * kLog2e;
            const float last2 = __shfl(incl, kWave - 1, kWave) * kLog2e;
            float* cum2 = fcum2(buf);
            // this wave's quarter of the tokens: lanes [16 sw, 16 sw + 16)
            const bool mine = lane / 16 == sw;
            if (mine) {
#pragma unroll
                for (int j = 0; j < LA; ++j) cum2[lane * LA + j] = cum[j];
            }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this wave reads back what it wrote
            if (mine) {
#pragma unroll
                for (int j = 0; j < LA; ++j) {
                    const int t = lane * LA + j;
                    fu(buf)[t] = fexp2(cum2[t | 15] - cum[j]);
                    ff(buf)[t] = fexp2(cum[j] - cum2[t & ~15]);
                    fw(buf)[t] = fexp2(last2 - cum[j]);
                }
            }
            if (sw == 0) {
                // block boundary sums straight from the lanes that hold them
                const float a2 = __shfl(cum[0], (16 * (lane / NT)) / LA, kWave);
                const float e2 = __shfl(cum[LA - 1], (16 * (lane % NT) + 15) / LA, kWave);
                if (lane < NT * NT) fbeta(buf)[lane] = (lane % NT) < (lane / NT) ? fexp2(a2 - e2) : 0.f;
                const float s2 = __shfl(cum[0], (16 * lane) / LA, kWave);
                if (lane < NT) fea(buf)[lane] = fexp2(s2);
            }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __bf16* xsm = Xs + buf * Q * kXStr;
            __bf16* xwm = Xw + buf * Q * kXStr;
            const float* wrow = fw(buf);
#pragma unroll
            for (int m = 0; m < XCH; ++m) {
                const int id = lane + kWave * m, row = QW * sw + id / 8, c16 = id % 8;
                const uint4 raw = row < len ? xs[m] : zero;
                st16(xsm + row * kXStr + 8 * c16, raw);
                const float w = wrow[row];
                const bf16x8 rv = as_bf16x8(raw);
                bf16x8 sv;
#pragma unroll
                for (int j = 0; j < 8; ++j) sv[j] = (__bf16)((float)rv[j] * w);
                *reinterpret_cast<bf16x8*>(xwm + row * kXStr + 8 * c16) = sv;
            }
            return fexp2(last2);
        };

        f32x4 hs[NBW][PB];
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                hs[jn][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (prm.init) {
                    const int n = 16 * (sw + 4 * jn) + 4 * lg;
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
                    const int n = 16 * (sw + 4 * jn) + 4 * lg;
                    store4(hsm + (16 * pb + l16) * HS + n, hs[jn][pb][0], hs[jn][pb][1], hs[jn][pb][2], hs[jn][pb][3]);
                }
        };

        load_lax(0);
        load_b(0);
        float el = prepare(0);
        load_lax(min(1, nchunks - 1));
        write_state(Hs);
        lds_barrier();

        for (int c = 0; c < nchunks; ++c) {
            const int cn = min(c + 1, nchunks - 1);
            const __bf16* xwm = Xw + (c & 1) * Q * kXStr;
            // H_k = exp(cum_last) H_{k-1} + B^T (w o X)
#pragma unroll
            for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) hs[jn][pb] *= el;
#pragma unroll
            for (int k = 0; k < KS; ++k)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    const bf16x8 xf = token_frag(xwm, kXStr, 16 * pb, k, lane);
#pragma unroll
                    for (int jn = 0; jn < NBW; ++jn) hs[jn][pb] = mfma_bf16(as_bf16x8(bt[jn][k]), xf, hs[jn][pb]);
                }
            load_b(cn);
            write_state(Hs + ((c + 1) & 1) * kP * HS);
            if (c + 1 < nchunks) {
                el = prepare(c + 1);
                load_lax(min(c + 2, nchunks - 1));
            }
            lds_barrier();
        }

        if (prm.final_state) {
#pragma unroll
            for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    const int n = 16 * (sw + 4 * jn) + 4 * lg;
                    float* dst = prm.final_state + (unit * N + n) * kP + 16 * pb + l16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[i * kP] = hs[jn][pb][i];
                }
        }
    }
}

template <int N, int Q>
constexpr size_t prep_lds() {
    return (size_t)2 * Q * (N + 8) * 2;
}

// Lets a kernel use the full 160 KiB of LDS (once per device).
bool allow_full_lds(const void* kernel, bool* done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    if (!done[dev]) {
        if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) != hipSuccess)
            return false;
        done[dev] = true;
    }
    return true;
}

template <int N, int Q>
int launch_fast_t(const ForwardLaunch& fl, hipStream_t stream) {
    constexpr int NPAIR = n_pairs(Q / 16);
    static_assert(WalkShape<N, Q>::lds_bytes <= kMaxLds, "walk LDS budget");
    static bool prep_attr[64] = {}, walk_attr[64] = {};
    __bf16* pairs = reinterpret_cast<__bf16*>(fl.scores);
    const int64_t nblk = fl.batch * fl.ngroups * fl.nchunks;
    __bf16* bt = pairs + nblk * NPAIR * 512;
    PrepParams pp{fl.Bm, fl.Cm, pairs, bt, fl.seqlen, fl.ngroups, fl.nchunks};
    if (!allow_full_lds(reinterpret_cast<const void*>(&prep_kernel<N, Q>), prep_attr)) return -1;
    if (!allow_full_lds(reinterpret_cast<const void*>(&walk5_kernel<N, Q>), walk_attr)) return -1;
    if (!record_event(fl, 0, stream)) return -1;
    const size_t plds = prep_lds<N, Q>();
    hipLaunchKernelGGL((prep_kernel<N, Q>), dim3((unsigned)(nblk * kPrepParts)), dim3(kThreads), plds, stream, pp);
    if (hipGetLastError() != hipSuccess) return -1;

    const int64_t units = fl.batch * fl.nheads;
    const int64_t per_xcd = (units + 7) / 8;
    Walk2Params wp{fl.x, fl.log_a, fl.Cm, fl.D, pairs, bt, fl.init, fl.y, fl.final_state,
                   fl.batch, fl.seqlen, fl.nheads, fl.ngroups, fl.nchunks, per_xcd};
    if (!record_event(fl, 1, stream)) return -1;
    const size_t wlds = WalkShape<N, Q>::lds_bytes;
    hipLaunchKernelGGL((walk5_kernel<N, Q>), dim3((unsigned)(8 * per_xcd)), dim3(kWalkThreads), wlds, stream, wp);
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
