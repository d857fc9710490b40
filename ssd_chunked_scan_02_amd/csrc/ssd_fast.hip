// Pipelined chunk walk for bf16 inputs, scalar decay, head dim 64 (the Mamba-2 layer
// shape), gfx950.  Same operator as walk_kernel in ssd_kernels.hip (aiwiki "State Space
// Duality", "Two algorithms for one operator"; llms.blog "The Chunk-Wise SSD Algorithm"),
// organised for latency hiding and a small VALU budget:
//
//   prep_kernel   per (batch, group, chunk): the causal score tiles S^T = B C^T as bf16
//                 "pairs" (two 16x16 tiles along s) and the B^T MFMA operand fragments, both
//                 stored in the lane order the walk reads them, so each is one coalesced
//                 16-byte load per lane.
//   walk_fast_kernel  one workgroup (12 waves, three roles) per (batch, head) walks the chunks
//                 with the fp32 N x P state in registers.  Every global operand of chunk c+1
//                 is loaded into registers right after its last use in chunk c (one register
//                 set, rolling), and the one workgroup barrier per chunk orders LDS only, so
//                 those loads stay in flight across it.  x is staged row-major in LDS and read
//                 as MFMA operands that contract over tokens with the transposing LDS read
//                 ds_read_b64_tr_b16 (a 16-lane group whose lane 4j+q points at row r_j,
//                 columns 4q..4q+3 returns in lane i column i of rows r_0..r_3).
//
// Token order inside a 32-token MFMA step: lane group g, element j holds token
//   kperm(g, j) = 4g + j (j < 4),  16 + 4g + (j - 4) (j >= 4),
// the row set an accumulator lane of two stacked 16x16 tiles owns, so masked scores feed the
// intra-chunk product straight from registers.
//
// Decay mask without an exp per score: for a 16-token output block tb starting at token a
// and any token s before that block, exp(cum_t - cum_s) = f_t * U(tb, s) with
//   f_t = exp(cum_t - cum_a),  U(tb, s) = exp(cum_a - cum_s),
// both exp of a non-positive number; U is one table per chunk, so a masked score costs one
// multiply.  Only the 16x16 diagonal block of each output block takes exact exps.

#include <cmath>

#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Token flags of a packed batch walked as one sequence (Walk2Params::tok_flags): a token with
// either bit set begins a new stretch of the recurrence (a sequence start, or a token of no
// sequence, which stands alone).  Two tokens of one chunk share a sequence exactly when the number
// of such tokens up to each of them is the same.  Tag of a token outside every sequence: its count
// plus this (exact in fp32; counts are below 257).
constexpr int kFlagStart = 1, kFlagDead = 2;
// offsets of a packed batch that the prep kernel can stage in LDS to mark the tokens itself
// (more sequences take a marking launch of their own)
constexpr int kMarkLdsMax = 4096;
constexpr int kP = 64;            // head dim handled here
constexpr int kXStr = kP + 8;     // LDS row stride of the x tile, elements
constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ constexpr int pair_base(int tb) {
    return (tb % 2 == 0) ? (tb / 2) * (tb / 2 + 1) : (tb / 2 + 1) * (tb / 2 + 1);
}
__host__ __device__ constexpr int n_pairs(int nt) { return pair_base(nt); }
__device__ __forceinline__ int kperm(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

__device__ __forceinline__ v4i16 lds_read_tr(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
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
// prep_kernel: per (batch, group, chunk) one workgroup, or two when that many still fit on the
// CUs in one round (see below).  It reads the chunk's B and C rows once, stages them in LDS (rows
// past the sequence end as zeros) and writes
//   pairs[(b,g,c)][pair(tb,k)][lane][8]: S^T[32k + kperm(lg, j)][16 tb + l16] (0 where the
//       second tile lies above the diagonal), pair(tb,k) = pair_base(tb) + k, 2k <= tb;
//   ct[(b,g,c)][tb][k][lane][8]: C[16 tb + l16][32k + 8 lg + j]  (the C^T operand);
//   btf[(b,g,c)][nb][k][lane][8]: B[32k + kperm(lg, j)][16 nb + l16]  (the B^T operand);
//   la_t[b][h][c Q + t] = log a[b][c Q + t][h] for the group's heads (0 past the sequence
//       end), so the walk reads a head's chunk contiguously.
// waves of one prep workgroup: 16, or fewer when the chunk has fewer 16-byte pieces of B
template <int N, int Q> struct PrepShape {
    static constexpr int WAVES = Q * N / 8 / kWave < 16 ? Q * N / 8 / kWave : 16;
    static constexpr int THREADS = WAVES * kWave;
};
// log a items (head, 4 tokens) per prep thread: heads per group up to kPrepLa * 4 * 512 / chunk
// (the smallest prep workgroup has 512 threads)
constexpr int kPrepLa = 4;
constexpr int64_t kPrepSplitMax = 256;  // prep workgroups one round of the CUs holds
constexpr int kPrepMinThreads = 512;

// Ranks of a packed batch's (at most kOrderMax) sequences by length, longest first (ties by
// index): order[rank] = b.  Workgroup w of the ranking ranks sequences w THREADS .. + THREADS - 1,
// one per thread: it stages every length in LDS (lens, padded with -1 to a multiple of 4, which
// count for nothing), and each thread counts the sequences ahead of its own, four lengths per LDS
// read, every lane reading the same ones.
constexpr int64_t kOrderMax = 4096;
template <int THREADS>
__device__ void rank_sequences(const int64_t* seq_off, int64_t nseq, int64_t seqlen, int64_t total, int* order,
                               int* lens, int w, int tid) {
    const int n4 = (int)((nseq + 3) / 4);
    for (int64_t j = tid; j < 4 * (int64_t)n4; j += THREADS)
        lens[j] = j < nseq ? (int)seq_span(seq_off, j, seqlen, total).len : -1;
    __syncthreads();
    const int64_t i = (int64_t)w * THREADS + tid;
    if (i >= nseq) return;
    const int li = lens[i];
    int rank = 0;
    for (int j4 = 0; j4 < n4; ++j4) {
        const int4 v = reinterpret_cast<const int4*>(lens)[j4];
        const int j = 4 * j4;
        rank += (v.x > li || (v.x == li && j < (int)i)) ? 1 : 0;
        rank += (v.y > li || (v.y == li && j + 1 < (int)i)) ? 1 : 0;
        rank += (v.z > li || (v.z == li && j + 2 < (int)i)) ? 1 : 0;
        rank += (v.w > li || (v.w == li && j + 3 < (int)i)) ? 1 : 0;
    }
    order[rank] = (int)i;
}
// workgroups of the ranking, rounded up to a whole number of XCD rounds (8)
template <int THREADS>
constexpr int64_t ranking_groups(int64_t nseq) {
    return (nseq + 8 * THREADS - 1) / (8 * THREADS) * 8;
}

template <int N, int Q>
__global__ void __launch_bounds__((PrepShape<N, Q>::THREADS)) prep_kernel(PrepParams prm) {
    constexpr int kPrepThreads = PrepShape<N, Q>::THREADS, kPrepWaves = PrepShape<N, Q>::WAVES;
    constexpr int NT = Q / 16, KS = Q / 32, NB = N / 16, KN = N / 32;
    constexpr int NPAIR = n_pairs(NT);
    constexpr int NS = N + 8;
    constexpr int ITEMS = Q * (N / 8) / kPrepThreads;  // 16-byte pieces of B (and of C) per thread
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Bs = reinterpret_cast<__bf16*>(smem);   // [Q][NS]
    __bf16* Cs = Bs + Q * NS;                       // [Q][NS]
    const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, lg = lane / 16;
    // A packed batch's first workgroups (a whole number of XCD rounds, dispatched first so that
    // they overlap the blocks) rank its sequences for the walk's order, beside the blocks rather
    // than in a launch of their own before them.
    int64_t bid = blockIdx.x;
    if (prm.order) {
        const int64_t nseq = prm.nblk / (prm.ngroups * prm.nchunks), nrank = ranking_groups<kPrepThreads>(nseq);
        if (bid < nrank) {
            rank_sequences<kPrepThreads>(prm.seq_off, nseq, prm.seqlen, prm.total, prm.order,
                                         reinterpret_cast<int*>(smem), (int)bid, tid);
            return;
        }
        bid -= nrank;
    }
    // With prm.split, two workgroups per block on the same XCD (workgroup i runs on XCD i % 8),
    // which shortens the chain each one waits through: part 0 writes the score pairs, part 1 the
    // C^T and B^T fragments and log a head-major.  Otherwise one workgroup does all of it.
    const int part = prm.split ? (int)((bid / 8) % 2) : -1;
    const int64_t blk = prm.split ? (bid / 16) * 8 + bid % 8 : bid;
    if (blk >= prm.nblk) return;
    const bool do_pairs = part != 1, do_rest = part != 0;
    const int c = (int)(blk % prm.nchunks);
    const int64_t bg = blk / prm.nchunks;
    const int64_t b = bg / prm.ngroups, g = bg % prm.ngroups;
    const int64_t t0 = (int64_t)c * Q;
    const SeqSpan sq = seq_span(prm.seq_off, b, prm.seqlen, prm.total);
    if (t0 >= sq.len) return;  // (a packed sequence shorter than seqlen: no such chunk)
    const int len = (int)min((int64_t)Q, sq.len - t0);
    const int64_t rs = prm.ngroups * N;
    const __bf16* Bg = static_cast<const __bf16*>(prm.Bm) + ((sq.row0 + t0) * prm.ngroups + g) * N;
    const __bf16* Cg = static_cast<const __bf16*>(prm.Cm) + ((sq.row0 + t0) * prm.ngroups + g) * N;
    const uint4 zero = {0u, 0u, 0u, 0u};

    // every global load first, so one wait covers them all
    uint4 vb[ITEMS], vc[ITEMS];
#pragma unroll
    for (int m = 0; m < ITEMS; ++m) {
        const int id = tid + kPrepThreads * m, row = id / (N / 8), c8 = id % (N / 8);
        const int64_t off = min(row, len - 1) * rs + 8 * c8;
        vb[m] = ld16(Bg + off);
        vc[m] = ld16(Cg + off);
    }
    // (a packed batch walked as one sequence: its offsets, clamped into [0, total] as the
    // sequence-by-sequence walk clamps them, for the token flags of this chunk)
    const bool do_mark = prm.flags && do_rest && g == 0;
    constexpr int MO = (kMarkLdsMax + kPrepThreads - 1) / kPrepThreads;
    int mo[MO];
    if (do_mark) {
#pragma unroll
        for (int i = 0; i < MO; ++i) {
            const int64_t j = tid + (int64_t)kPrepThreads * i;
            const int64_t v = j <= prm.mark_nseq ? prm.mark_off[j] : 0;
            mo[i] = (int)(v < 0 ? 0 : (v > prm.total ? prm.total : v));
        }
    }
    if (do_rest) {
        // log a head-major: item (head, 4 tokens) gathers 4 rows (consecutive threads read
        // consecutive heads of a row) and writes 16 contiguous bytes; rows clamped, masked below
        // (with the discretisation front-end the same items read dt, laid out as log a, and
        // turn it into log a and log2 of the input scale)
        const int HG = (int)(prm.nheads / prm.ngroups);
        const int nla = HG * (Q / 4);
        const float* lag = (prm.dt ? prm.dt : prm.log_a) + (sq.row0 + t0) * prm.nheads + g * HG;
        const int wave0 = tid - lane;  // first thread of this wave
        f32x4 lv[kPrepLa];
#pragma unroll
        for (int i = 0; i < kPrepLa; ++i) {
            if (wave0 + kPrepThreads * i >= nla) continue;  // (uniform over the wave)
            const int id = min(tid + kPrepThreads * i, nla - 1), hl = id % HG, t4 = 4 * (id / HG);
#pragma unroll
            for (int j = 0; j < 4; ++j) lv[i][j] = lag[(int64_t)min(t4 + j, len - 1) * prm.nheads + hl];
        }
        {
            const int64_t tpad = (int64_t)prm.nchunks * Q;
            const int64_t off0 = (b * prm.nheads + g * HG) * tpad + t0;
            float* dst = prm.la_t + off0;
#pragma unroll
            for (int i = 0; i < kPrepLa; ++i) {
                const int id = tid + kPrepThreads * i, hl = id % HG, t4 = 4 * (id / HG);
                if (wave0 + kPrepThreads * i >= nla) continue;
                f32x4 v, lgv = {0.f, 0.f, 0.f, 0.f};
                if (prm.dt) {
                    // log a = -softplus(dt + bias) exp(A_log), and log2 softplus(dt + bias)
                    const int64_t hh = g * HG + min(id, nla - 1) % HG;
                    const float bias = prm.dt_bias ? prm.dt_bias[hh] : 0.f;
                    const float ea = expf(prm.A_log[hh]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float u = lv[i][j] + bias;
                        const float sp = softplus_hw(u);
                        v[j] = t4 + j < len ? -sp * ea : 0.f;
                        lgv[j] = t4 + j < len ? log2_softplus_hw(u, sp) : 0.f;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = t4 + j < len ? lv[i][j] : 0.f;
                }
                if (id < nla) {
                    *reinterpret_cast<f32x4*>(dst + hl * tpad + t4) = v;
                    if (prm.lg_t) *reinterpret_cast<f32x4*>(prm.lg_t + off0 + hl * tpad + t4) = lgv;
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < ITEMS; ++m) {
        const int id = tid + kPrepThreads * m, row = id / (N / 8), c8 = id % (N / 8);
        st16(Bs + row * NS + 8 * c8, row < len ? vb[m] : zero);
        st16(Cs + row * NS + 8 * c8, row < len ? vc[m] : zero);
    }
    int* offs = reinterpret_cast<int*>(Cs + Q * NS);  // [mark_nseq + 1]
    if (do_mark) {
#pragma unroll
        for (int i = 0; i < MO; ++i) {
            const int j = tid + kPrepThreads * i;
            if (j <= prm.mark_nseq) offs[j] = mo[i];
        }
    }
    __syncthreads();
    if (do_mark && tid < Q) {
        // Token t of the packed axis: outside every sequence before the first offset and from the
        // last one on; otherwise in sequence a, the last one starting at or before t (offsets are
        // non-decreasing, so a nonempty one), which it starts when t is its first token and which
        // has left it behind when t lies past its first mark_bound tokens.  (Malformed offsets
        // give wrong flags, and every read stays inside [0, mark_nseq].)  Tokens past the packed
        // axis, in the last chunk's tail, stay 0.
        const int64_t t = t0 + tid;
        const int nseq = (int)prm.mark_nseq;
        int flag = 0;
        if (t < prm.total) {
            if (t < offs[0] || t >= offs[nseq]) {
                flag = kFlagStart | kFlagDead;
            } else {
                int a = 0, z = nseq;  // offs[a] <= t < offs[z] for well-formed offsets
                while (z - a > 1) {
                    const int m = (a + z) >> 1;
                    if (offs[m] <= t) a = m;
                    else z = m;
                }
                const int64_t s0 = offs[a];
                if (t == s0) flag = kFlagStart;
                if (t - s0 >= prm.mark_bound) flag = kFlagStart | kFlagDead;
            }
        }
        prm.flags[t] = flag;
    }

    if (do_rest) {
        __bf16* ct = prm.ct + blk * (int64_t)NT * KN * 512 + lane * 8;
        for (int f = wave; f < NT * KN; f += kPrepWaves) {
            const int tb = f / KN, k = f % KN;
            st16(ct + f * 512, ld16(Cs + (16 * tb + l16) * NS + 32 * k + 8 * lg));
        }
        __bf16* btf = prm.bt + blk * (int64_t)NB * KS * 512 + lane * 8;
        for (int f = wave; f < NB * KS; f += kPrepWaves) {
            const int nb = f / KS, k = f % KS;
            *reinterpret_cast<bf16x8*>(btf + f * 512) = token_frag(Bs, NS, 16 * nb, k, lane);
        }
    }
    if (!do_pairs) return;
    __bf16* pairs = prm.pairs + blk * (int64_t)NPAIR * 512 + lane * 8;
    for (int idx = wave; idx < NPAIR; idx += kPrepWaves) {
        int tb = 0;
        while (pair_base(tb + 1) <= idx) ++tb;
        const int k = idx - pair_base(tb);
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int sb = 2 * k + hh;
            if (sb > tb) continue;
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
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
// walk_fast_kernel: 12 waves per (batch, head) in three roles; wave i runs on SIMD i % 4, so
// each SIMD interleaves one wave of each role (three waves per SIMD, at most 168 VGPRs each).
// Each role body is compiled once per wave index, so every causal branch and block index below
// is resolved at compile time.
//   output waves 0-3: y of their 16-token blocks for chunk c, from H_{k-1} (LDS), the staged
//       x and decay factors of chunk c, C rows and score pairs (registers); y staged in LDS.
//   state waves 4-7: H_k = exp(cum_last) H_{k-1} + B^T (w o X) for chunk c, written to the
//       other LDS state buffer.
//   helper waves 8-11: chunk c+1 for everyone (running sums of log a by a wave-wide DPP scan,
//       decay factors, x staged raw and weighted by w) and the stores of chunk c-1's y.
// One LDS barrier per chunk; everything written for chunk c+1 goes to the other of two
// buffers (y: staged for chunk c, stored during chunk c+1), whose previous contents every wave
// finished before the last barrier.  (Two roles, with the state waves also doing the helpers'
// work and the output waves storing y, took 42.1-44.3 us for the walk at the Mamba-2 layer
// shape; three roles 41.9-42.0 us.)
//
// Global addresses are a wave-uniform 64-bit base per chunk plus a 32-bit per-lane byte
// offset (the host only takes this path when every offset inside a chunk fits).
constexpr int kWalkWaves = 12;
// workgroups of a segmented fast walk: one round (one per CU).  Two rounds of half as long
// segments give the state pass more workgroups but measured slower at the long-sequence workload
// (255-258 against 249-253 us per forward: walk 175 against 169 us, state pass 31 against 36.5 us).
constexpr int64_t kSegTarget = 256;
// bytes of x above which the walk reads x with streaming loads (the MI355X last-level cache is 256 MB)
constexpr double kXStreamBytes = 128.0 * 1024 * 1024;
constexpr int kWalkThreads = kWalkWaves * kWave;

// 16-token block handled by output wave `ow` in its r-th round (snake order balances the
// causal work across the four output waves).
__host__ __device__ constexpr int wave_tb(int r, int ow) { return (r % 2 == 0) ? 4 * r + ow : 4 * r + 3 - ow; }

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

// (token flags: see kFlagStart)
constexpr float kDeadTag = 65536.f;
// log2 decay that stands for "the recurrence restarts here": exp2 of it is 0, and it stays hugely
// negative under the additions of ordinary decays.
constexpr float kRestart2 = -1.0e30f;

__device__ __forceinline__ float lane_value(float v, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 32; o > 0; o /= 2) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

// 16-byte global load at a uniform base plus a per-lane byte offset.
__device__ __forceinline__ uint4 ldg16(const void* base, uint32_t off) {
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + off);
}

// Raw buffer resource over `bytes` bytes at `base`: buffer stores at or past that many bytes
// are dropped by the hardware range check, which masks a short chunk's tail rows without a
// branch.  The last word is the gfx9 default format (32-bit data, no swizzle).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 16-byte store through a buffer resource, marked non-temporal (streaming; cache-policy bit 1):
// for outputs nothing reads back, so that they do not take L2 lines from the operands the heads
// of a group share (C2 walk 44.6 -> 40.8 us against plain stores).
__device__ __forceinline__ void buffer_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 2);
}
// 16-byte global load marked non-temporal (streaming): the line is taken into the caches at the
// lowest priority, so that a stream read once does not evict what other waves read again.
__device__ __forceinline__ uint4 ldg16_stream(const void* base, uint32_t off) {
    return __builtin_bit_cast(
        uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + off)));
}
// 16-byte load through a buffer resource; reads at or past its size return zeros.
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Orders this wave's LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

template <int N, int Q>
struct WalkShape {
    static constexpr int NT = Q / 16, TBW = NT / 4, KS = Q / 32, KN = N / 32, NBW = N / 64;
    static constexpr int LA = Q / 64, QW = Q / 4, XCH = QW * 8 / kWave, NPAIR = n_pairs(NT);
    static constexpr int PB = kP / 16, HS = N + 8;
    // one decay-factor buffer, floats: cum2 [Q] (log2 e times the running sum of log a),
    // f [Q], w [Q], U [NT][Q], ea [NT], cs2 [Q] (the running sums on the input side of a
    // factor: cum2 - log2 of the input scale, written only with one), tag [Q] (a packed batch
    // walked as one sequence: the count of sequence starts up to each token, plus kDeadTag for a
    // token outside every sequence; written only then)
    // el [4]: exp(cum_last) in its first float (the state's decay over the chunk), padded
    static constexpr int FSZ = 5 * Q + NT * Q + NT + 4;
    static constexpr int YROWS = 16 * TBW;  // output rows of one output wave per chunk
    static constexpr size_t lds_bytes =
        (size_t)(4 * Q * kXStr + 2 * kP * HS + 8 * YROWS * kXStr) * 2 + (size_t)2 * FSZ * 4;
};

// Factors of one chunk, with cum the running sum of log a inside the chunk (inclusive),
// a = 16 tb the first token of block tb and e the last token of the chunk:
//   f[t]     = exp(cum_t - cum_{a(t)}), a(t) the first token of t's block   (<= 1)
//   w[s]     = exp(cum_e - cum_s)                                            (<= 1)
//   U[tb][s] = exp(cum_a - cum_s) for s < a, else 0                          (<= 1)
//   ea[tb]   = exp(cum_a)                                                    (<= 1)
// so that exp(cum_t - cum_s) = f[t] U[tb][s] for s before t's block and exp(cum_t) = f[t] ea[tb].
template <int N, int Q>
struct WalkLds {
    using WS = WalkShape<N, Q>;
    __bf16* Xs;  // [2][Q][kXStr] x
    __bf16* Xw;  // [2][Q][kXStr] w o x
    __bf16* Hs;  // [2][kP][HS] H^T, bf16
    __bf16* Ys;  // [2][4][YROWS][kXStr] each output wave's rows of y by chunk parity, staged for full-row stores
    float* Fs;   // [2][FSZ]
    __device__ explicit WalkLds(unsigned char* smem) {
        Xs = reinterpret_cast<__bf16*>(smem);
        Xw = Xs + 2 * Q * kXStr;
        Hs = Xw + 2 * Q * kXStr;
        Ys = Hs + 2 * kP * WS::HS;
        Fs = reinterpret_cast<float*>(Ys + 8 * WS::YROWS * kXStr);
    }
    __device__ float* cum2(int buf) const { return Fs + buf * WS::FSZ; }
    __device__ float* f(int buf) const { return Fs + buf * WS::FSZ + Q; }
    __device__ float* w(int buf) const { return Fs + buf * WS::FSZ + 2 * Q; }
    __device__ float* U(int buf) const { return Fs + buf * WS::FSZ + 3 * Q; }
    __device__ float* ea(int buf) const { return Fs + buf * WS::FSZ + 3 * Q + WS::NT * Q; }
    __device__ float* cs2(int buf) const { return Fs + buf * WS::FSZ + 3 * Q + WS::NT * Q + WS::NT; }
    __device__ float* tag(int buf) const { return Fs + buf * WS::FSZ + 4 * Q + WS::NT * Q + WS::NT; }
    __device__ float* el(int buf) const { return Fs + buf * WS::FSZ + 5 * Q + WS::NT * Q + WS::NT; }
};

// The piece of work of one workgroup: a (batch, head) unit and the chunks [c0, c1) of one
// segment of its sequence (the whole sequence unless the walk is split into segments); the
// sequence's first row, length and chunk count (a packed sequence: its own).
struct WalkSpan {
    int64_t unit, b, h, g, row0, len;
    int seg, c0, c1, nch;
};

__device__ __forceinline__ WalkSpan walk_span(const Walk2Params& prm, int64_t work, int Q) {
    WalkSpan sp;
    const int64_t units = prm.batch * prm.nheads;
    sp.seg = (int)(work / units);
    sp.unit = work % units;
    sp.b = sp.unit / prm.nheads;
    sp.h = sp.unit % prm.nheads;
    sp.g = sp.h / (prm.nheads / prm.ngroups);
    const SeqSpan sq = seq_span(prm.seq_off, sp.b, prm.seqlen, prm.total);
    sp.row0 = sq.row0;
    sp.len = sq.len;
    sp.nch = prm.seq_off ? (int)((sq.len + Q - 1) / Q) : prm.nchunks;
    sp.c0 = sp.seg * prm.seg_chunks;
    sp.c1 = min(sp.c0 + prm.seg_chunks, sp.nch);
    return sp;
}

template <int N, int Q, int OW, bool DT, bool PK>
__device__ __forceinline__ void walk_output_role(const Walk2Params& prm, const WalkLds<N, Q>& L, const WalkSpan& span,
                                                 int lane) {
    const int64_t b = span.b, h = span.h, g = span.g;
    const int c0 = span.c0, c1 = span.c1;
    using WS = WalkShape<N, Q>;
    constexpr int NT = WS::NT, TBW = WS::TBW, KS = WS::KS, KN = WS::KN, NPAIR = WS::NPAIR;
    constexpr int PB = WS::PB, HS = WS::HS;
    constexpr int KDMAX = wave_tb(TBW - 1, OW) / 2 > wave_tb(0, OW) / 2 ? wave_tb(TBW - 1, OW) / 2 : wave_tb(0, OW) / 2;
    const int l16 = lane % 16, lg = lane / 16;
    const int64_t G = prm.ngroups;
    const int nchunks = prm.nchunks;
    const __bf16* ct0 = prm.ct + (b * G + g) * (int64_t)nchunks * NT * KN * 512;
    const __bf16* pairs0 = prm.pairs + (b * G + g) * (int64_t)nchunks * NPAIR * 512;
    const float dskip = prm.D ? prm.D[h] : 0.f;
    constexpr int YROWS = WS::YROWS;

    // Operands come from the prep kernel in lane order (one contiguous 1 KiB per load); rows
    // past a short chunk's end are zeros there and are never stored here.
    uint4 cf[TBW][KN], sp[TBW][KS];
    auto load_c = [&](int c) {
        const void* base = ct0 + (int64_t)c * NT * KN * 512;
#pragma unroll
        for (int r = 0; r < TBW; ++r)
#pragma unroll
            for (int k = 0; k < KN; ++k) cf[r][k] = ldg16(base, 16 * lane + (wave_tb(r, OW) * KN + k) * 1024);
    };
    auto load_s = [&](int c) {
        const void* base = pairs0 + (int64_t)c * NPAIR * 512;
#pragma unroll
        for (int r = 0; r < TBW; ++r) {
            const int tb = wave_tb(r, OW);
#pragma unroll
            for (int k = 0; k <= tb / 2; ++k) sp[r][k] = ldg16(base, 16 * lane + (pair_base(tb) + k) * 1024);
        }
    };
    // inside a diagonal block, token 4 lg + j against token l16
    bool causal[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) causal[j] = 4 * lg + j <= l16;

    load_c(c0);
    load_s(c0);
    lds_barrier();

    for (int c = c0; c < c1; ++c) {
        const int cn = min(c + 1, c1 - 1);
        const int buf = c & 1;
        const __bf16* xsm = L.Xs + buf * Q * kXStr;
        const __bf16* hcur = L.Hs + buf * kP * HS;
        const float* cum2 = L.cum2(buf);
        const float* cin2 = DT ? L.cs2(buf) : cum2;  // input side of the in-block factors
        const float* ffa = L.f(buf);
        const float* Ut = L.U(buf);
        const float* ea = L.ea(buf);
        const float* tagr = L.tag(buf);
        __bf16* ys = L.Ys + (buf * 4 + OW) * YROWS * kXStr;  // (the helper waves store it next chunk)

        // carried state: acc = exp(cum_a) C_t H_{k-1}  (acc rows: p, columns: t)
        f32x4 acc[TBW][PB];
#pragma unroll
        for (int r = 0; r < TBW; ++r)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[r][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // (operands read step by step: with three waves per SIMD the other waves cover the LDS
        // latency, and the registers stay under the 168 that three waves allow)
#pragma unroll
        for (int k = 0; k < KN; ++k) {
            bf16x8 hk[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) hk[pb] = as_bf16x8(ld16(hcur + (16 * pb + l16) * HS + 32 * k + 8 * lg));
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int r = 0; r < TBW; ++r) acc[r][pb] = mfma_bf16(hk[pb], as_bf16x8(cf[r][k]), acc[r][pb]);
        }
        load_c(cn);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch here, a chunk ahead of its use
#pragma unroll
        for (int r = 0; r < TBW; ++r) {
            const float sc = ea[wave_tb(r, OW)];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) acc[r][pb] *= sc;
        }

        // inside the chunk: (S o L) X over the 32-token steps
#pragma unroll
        for (int k = 0; k <= KDMAX; ++k) {
            bf16x8 xf[PB];
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) xf[pb] = token_frag(xsm, kXStr, 16 * pb, k, lane);
#pragma unroll
            for (int r = 0; r < TBW; ++r) {
                const int tb = wave_tb(r, OW);
                const int kd = tb / 2;  // the step holding the diagonal block
                if (k > kd) continue;
                float s8[8];
                unpack8(as_bf16x8(sp[r][k]), s8);
                bf16x8 bop;
                if (k < kd) {
                    const f32x4 u0 = *reinterpret_cast<const f32x4*>(Ut + tb * Q + 32 * k + 4 * lg);
                    const f32x4 u1 = *reinterpret_cast<const f32x4*>(Ut + tb * Q + 32 * k + 16 + 4 * lg);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        bop[j] = (__bf16)(s8[j] * u0[j]);
                        bop[j + 4] = (__bf16)(s8[j + 4] * u1[j]);
                    }
                } else {
                    // the remaining factor f_t first; then the diagonal block with exact exps
                    // (and for an odd block, the block before it through U)
                    const int t = 16 * tb + l16;
                    const float ft = ffa[t];
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) acc[r][pb] *= ft;
                    const float ct = cum2[t];
                    const f32x4 cd = *reinterpret_cast<const f32x4*>(cin2 + 16 * tb + 4 * lg);
                    // (a packed batch: only pairs of one sequence)
                    bool keep[4];
                    if constexpr (PK) {
                        const float tt = tagr[t];
                        const f32x4 ts = *reinterpret_cast<const f32x4*>(tagr + 16 * tb + 4 * lg);
#pragma unroll
                        for (int j = 0; j < 4; ++j) keep[j] = causal[j] && ts[j] == tt;
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) keep[j] = causal[j];
                    }
                    if (tb % 2 == 0) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float v = s8[j] * fexp2(ct - cd[j]);
                            bop[j] = (__bf16)(keep[j] ? v : 0.f);
                            bop[j + 4] = (__bf16)0.f;
                        }
                    } else {
                        const f32x4 u0 = *reinterpret_cast<const f32x4*>(Ut + tb * Q + 32 * k + 4 * lg);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            bop[j] = (__bf16)(s8[j] * (ft * u0[j]));
                            const float v = s8[j + 4] * fexp2(ct - cd[j]);
                            bop[j + 4] = (__bf16)(keep[j] ? v : 0.f);
                        }
                    }
                }
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) acc[r][pb] = mfma_bf16(xf[pb], bop, acc[r][pb]);
            }
        }
        load_s(cn);
        __builtin_amdgcn_sched_barrier(0);

        // skip term; y through this wave's LDS rows, then stored as whole 128-byte rows (rows
        // past a short chunk's end fall outside the buffer resource and are dropped)
#pragma unroll
        for (int r = 0; r < TBW; ++r) {
            const int t = 16 * wave_tb(r, OW) + l16;
            // (no branch on D: a missing skip term adds 0 x; one path keeps the load counting exact)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                const bf16x4 x4 = *reinterpret_cast<const bf16x4*>(xsm + t * kXStr + 16 * pb + 4 * lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[r][pb][i] += dskip * (float)x4[i];
            }
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
                store4(ys + (16 * r + l16) * kXStr + 16 * pb + 4 * lg, acc[r][pb][0], acc[r][pb][1], acc[r][pb][2],
                       acc[r][pb][3]);
        }
        lds_barrier();
    }
}

// The helper waves of the walk: for chunk c + 1 the decay factors (running sums of log a, f, w, U,
// ea and the state's decay el) and x staged raw and weighted by w, while the other roles work on
// chunk c; and the y rows the output waves staged for chunk c - 1, stored as whole 128-byte rows.
// Helper wave SW takes the factors and x rows of the chunk's quarter SW and the y rows of output
// wave SW.  XS: x read with streaming loads (ldg16_stream).
template <int N, int Q, int SW, bool DT, bool PK, bool XS>
__device__ __forceinline__ void walk_helper_role(const Walk2Params& prm, const WalkLds<N, Q>& L, const WalkSpan& span,
                                                int lane) {
    const int64_t h = span.h, unit = span.unit;
    const int c0 = span.c0, c1 = span.c1;
    using WS = WalkShape<N, Q>;
    constexpr int NT = WS::NT, LA = WS::LA, QW = WS::QW, XCH = WS::XCH;
    const int64_t H = prm.nheads;
    const int nchunks = prm.nchunks;
    const uint32_t x_row = (uint32_t)(H * kP * 2);
    const float* la0 = prm.la_t + unit * (int64_t)nchunks * Q;
    const float* lg0 = DT ? prm.lg_t + unit * (int64_t)nchunks * Q : nullptr;
    const int* fl0 = PK ? prm.tok_flags : nullptr;
    const __bf16* xg = static_cast<const __bf16*>(prm.x);
    const uint4 zero = {0u, 0u, 0u, 0u};
    auto chunk_len = [&](int c) { return (int)min((int64_t)Q, span.len - (int64_t)c * Q); };

    float la[LA];
    float lgs[DT ? LA : 1];  // (DT) log2 of the input scale of the same tokens
    int flg[PK ? LA : 1];    // (PK) the token flags of the same tokens
    uint4 xs[XCH];
    // log a of the whole chunk (every helper wave scans it all) and x rows of this wave's
    // quarter of the chunk; rows clamped into the chunk, masked when staged.  Each is loaded
    // a full chunk ahead of its use.
    auto load_la = [&](int c) {
        const int64_t t0 = (int64_t)c * Q;
#pragma unroll
        for (int j = 0; j < LA; ++j) la[j] = la0[t0 + lane * LA + j];
        if (DT)
#pragma unroll
            for (int j = 0; j < LA; ++j) lgs[j] = lg0[t0 + lane * LA + j];
        if (PK)
#pragma unroll
            for (int j = 0; j < LA; ++j) flg[j] = fl0[t0 + lane * LA + j];
    };
    auto load_x = [&](int c) {
        const int last = chunk_len(c) - 1;
        const void* xbase = xg + ((span.row0 + (int64_t)c * Q) * H + h) * kP;
#pragma unroll
        for (int m = 0; m < XCH; ++m) {
            const int id = lane + kWave * m, row = min(QW * SW + id / 8, last), c16 = id % 8;
            const uint32_t off = (uint32_t)row * x_row + 16 * c16;
            xs[m] = XS ? ldg16_stream(xbase, off) : ldg16(xbase, off);
        }
    };
    // Decay factors of chunk c into factor buffer c & 1, with exp(cum_last) in its el slot.
    auto factors = [&](int c) {
        const int len = chunk_len(c);
        const int buf = c & 1;
        float cum[LA], run = 0.f;
#pragma unroll
        for (int j = 0; j < LA; ++j) { run += (lane * LA + j < len) ? la[j] : 0.f; cum[j] = run; }
        const float incl = wave_inclusive_sum(run);
        const float excl = incl - run;
#pragma unroll
        for (int j = 0; j < LA; ++j) cum[j] = (excl + cum[j]) * kLog2e;
        const float last2 = lane_value(incl, kWave - 1) * kLog2e;
        // running sum at the first token of this lane's 16-token block
        const float blk2 = __shfl(cum[0], lane & ~(16 / LA - 1), kWave);
        // the input side of each factor: with an input scale, exp2(c - cum_s) times the scale of
        // token s is exp2(c - (cum_s - log2 scale_s))
        float cin[LA];
#pragma unroll
        for (int j = 0; j < LA; ++j) cin[j] = DT ? cum[j] - lgs[j] : cum[j];
        // (PK) sequence tags: the running count of tokens that begin a new stretch of the
        // recurrence; every factor that links two tokens of different tags is 0, and so is the
        // decay of the state carried into the chunk past the first such token.  (Counts are
        // exact in fp32.)
        float cnt[LA];
        float cnt_e = 0.f, cnt_b = 0.f;
        if constexpr (PK) {
            float crun = 0.f;
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                crun += flg[j] != 0 ? 1.f : 0.f;
                cnt[j] = crun;
            }
            const float cincl = wave_inclusive_sum(crun);
#pragma unroll
            for (int j = 0; j < LA; ++j) cnt[j] += cincl - crun;
            cnt_e = lane_value(cincl, kWave - 1);
            cnt_b = __shfl(cnt[0], lane & ~(16 / LA - 1), kWave);
        }
        // this wave's quarter of the tokens: lanes [16 SW, 16 SW + 16)
        if (lane / 16 == SW) {
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const int t = lane * LA + j;
                L.cum2(buf)[t] = cum[j];
                if (DT) L.cs2(buf)[t] = cin[j];
                if constexpr (PK) {
                    L.f(buf)[t] = cnt[j] == cnt_b ? fexp2(cum[j] - blk2) : 0.f;
                    L.w(buf)[t] = cnt[j] == cnt_e ? fexp2(last2 - cin[j]) : 0.f;
                    L.tag(buf)[t] = cnt[j] + ((flg[j] & kFlagDead) ? kDeadTag : 0.f);
                } else {
                    L.f(buf)[t] = fexp2(cum[j] - blk2);
                    L.w(buf)[t] = fexp2(last2 - cin[j]);
                }
            }
        }
        // rows SW, SW + 4, ... of U
#pragma unroll
        for (int tb = SW; tb < NT; tb += 4) {
            const float ca = lane_value(cum[0], 16 * tb / LA);
            const float cnt_a = PK ? lane_value(cnt[0], 16 * tb / LA) : 0.f;
            float* urow = L.U(buf) + tb * Q;
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const int s = lane * LA + j;
                urow[s] = s < 16 * tb && (!PK || cnt[j] == cnt_a) ? fexp2(ca - cin[j]) : 0.f;
            }
        }
        if (SW == 0) {
            const float s2 = __shfl(cum[0], (16 * lane) / LA, kWave);
            const float c2 = PK ? __shfl(cnt[0], (16 * lane) / LA, kWave) : 0.f;
            if (lane < NT) L.ea(buf)[lane] = c2 == 0.f ? fexp2(s2) : 0.f;
        }
        if (SW == 0 && lane == 0) L.el(buf)[0] = cnt_e == 0.f ? fexp2(last2) : 0.f;
    };
    // x of chunk c into the x buffers c & 1, raw and weighted by w (after factors(c)).
    auto stage_x = [&](int c) {
        const int len = chunk_len(c);
        const int buf = c & 1;
        wave_lds_fence();  // this wave reads back the w it wrote
        __bf16* xsm = L.Xs + buf * Q * kXStr;
        __bf16* xwm = L.Xw + buf * Q * kXStr;
        const float* wrow = L.w(buf);
#pragma unroll
        for (int m = 0; m < XCH; ++m) {
            const int id = lane + kWave * m, row = QW * SW + id / 8, c16 = id % 8;
            const uint4 raw = row < len ? xs[m] : zero;
            st16(xsm + row * kXStr + 8 * c16, raw);
            const float w = wrow[row];
            const bf16x8 rv = as_bf16x8(raw);
            bf16x8 sv;
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[j] = (__bf16)((float)rv[j] * w);
            *reinterpret_cast<bf16x8*>(xwm + row * kXStr + 8 * c16) = sv;
        }
    };

    // y rows of output wave SW for chunk c, from its staging buffer (parity c & 1), as whole 128-byte
    // rows (rows past a short chunk's end fall outside the buffer resource and are dropped; with
    // `none` every store is dropped, which keeps one path through the loop)
    constexpr int TBW = WS::TBW, YROWS = WS::YROWS, YST = YROWS * 8 / kWave;
    const uint32_t y_row = (uint32_t)(H * kP * 2);
    __bf16* yg = static_cast<__bf16*>(prm.y);
    auto store_y = [&](int c, bool none) {
        const int len = chunk_len(c);
        const __bf16* ys = L.Ys + ((c & 1) * 4 + SW) * YROWS * kXStr;
        const float* tagr = L.tag(c & 1);
        const __amdgpu_buffer_rsrc_t yr =
            buffer_rsrc(yg + ((span.row0 + (int64_t)c * Q) * H + h) * kP, none ? 0u : (uint32_t)len * y_row);
#pragma unroll
        for (int m = 0; m < YST; ++m) {
            const int id = lane + kWave * m, row = id / 8, c8 = id % 8;
            const int t = 16 * wave_tb(row / 16, SW) + row % 16;
            // (a packed batch: rows outside every sequence are not written)
            if (!PK || tagr[t] < kDeadTag)
                buffer_store16_nt(yr, (uint32_t)t * y_row + 16 * c8, ld16(ys + row * kXStr + 8 * c8));
        }
    };
    (void)TBW;

    load_la(c0);
    load_x(c0);
    factors(c0);
    load_la(min(c0 + 1, c1 - 1));
    stage_x(c0);
    load_x(min(c0 + 1, c1 - 1));
    lds_barrier();

    // Per chunk: chunk c - 1's y (before its factor buffer, which holds the packed batch's tags, is
    // rewritten), the next chunk's factors and x staging, the loads a chunk ahead.  All of it runs
    // unconditionally (past the last chunk the next chunk's buffers get zeros nobody reads).
    for (int c = c0; c < c1; ++c) {
        store_y(c > c0 ? c - 1 : c0, c == c0);
        factors(c + 1);
        load_la(min(c + 2, c1 - 1));
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch here, a chunk ahead of its use
        stage_x(c + 1);
        load_x(min(c + 2, c1 - 1));
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
    }
    store_y(c1 - 1, false);
}

// The state waves of the walk: H_k = exp(cum_last) H_{k-1} + B^T (w o X) for chunk c, with the
// factors and w o x the helper waves staged, written to the other LDS state buffer.
template <int N, int Q, int SW, bool DT, bool PK>
__device__ __forceinline__ void walk_state_role(const Walk2Params& prm, const WalkLds<N, Q>& L, const WalkSpan& span,
                                                int lane) {
    const int64_t b = span.b, g = span.g, unit = span.unit;
    const int c0 = span.c0, c1 = span.c1;
    using WS = WalkShape<N, Q>;
    constexpr int KS = WS::KS, NBW = WS::NBW;
    constexpr int PB = WS::PB, HS = WS::HS;
    const int l16 = lane % 16, lg = lane / 16;
    const int64_t G = prm.ngroups;
    const int nchunks = prm.nchunks;
    const __bf16* bt0 = prm.bt + (b * G + g) * (int64_t)nchunks * (N / 16) * KS * 512;

    uint4 bt[NBW][KS];  // B^T operands, loaded a full chunk ahead of their use
    auto load_b = [&](int c) {
        const void* base = bt0 + (int64_t)c * (N / 16) * KS * 512;
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int k = 0; k < KS; ++k) bt[jn][k] = ldg16(base, 16 * lane + ((SW + 4 * jn) * KS + k) * 1024);
    };
    // The state entering the first chunk.  For segment s > 0 of a segmented walk it is the chain
    // h <- exp2(decay_j) h + state_j over the segments j < s (local states and log2 decays from
    // seg_state_kernel), started from the caller's initial state.  Where a factor exp2(decay_j)
    // is exactly 0 the chain restarts at state_j, whatever came before, so the chain is run from
    // the last such j: on long segments that is a single step.
    f32x4 hs[NBW][PB];
    auto add_rows = [&](const float* src, float scale) {
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int n = 16 * (SW + 4 * jn) + 4 * lg;
                const float* p = src + n * kP + 16 * pb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) hs[jn][pb][i] = scale * hs[jn][pb][i] + p[i * kP];
            }
    };
#pragma unroll
    for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) hs[jn][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const int64_t units = prm.batch * prm.nheads;
        int j0 = 0;
        bool restart = false;
        for (int j = span.seg - 1; j >= 0; --j)
            if (exp2f(prm.seg_decay[j * units + unit]) == 0.f) {
                j0 = j;
                restart = true;
                break;
            }
        if (!restart && prm.init) add_rows(prm.init + unit * N * kP, 0.f);
        for (int j = j0; j < span.seg; ++j)
            add_rows(prm.seg_state + (j * units + unit) * N * kP,
                     j == j0 && restart ? 0.f : exp2f(prm.seg_decay[j * units + unit]));
    }
    auto write_state = [&](__bf16* hsm) {
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int n = 16 * (SW + 4 * jn) + 4 * lg;
                store4(hsm + (16 * pb + l16) * HS + n, hs[jn][pb][0], hs[jn][pb][1], hs[jn][pb][2], hs[jn][pb][3]);
            }
    };

    load_b(c0);
    write_state(L.Hs + (c0 & 1) * kP * HS);
    lds_barrier();

    // Per chunk: the state MFMAs, the next chunk's B^T loads while they drain, then the state.
    for (int c = c0; c < c1; ++c) {
        const int cn = min(c + 1, c1 - 1);
        const __bf16* xwm = L.Xw + (c & 1) * Q * kXStr;
        const float el = L.el(c & 1)[0];
        // H_k = exp(cum_last) H_{k-1} + B^T (w o X)
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) hs[jn][pb] *= el;
        // every operand read issued before the first MFMA, so LDS latency is paid once
        bf16x8 xfa[KS][PB];
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) xfa[k][pb] = token_frag(xwm, kXStr, 16 * pb, k, lane);
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int jn = 0; jn < NBW; ++jn) hs[jn][pb] = mfma_bf16(as_bf16x8(bt[jn][k]), xfa[k][pb], hs[jn][pb]);
        load_b(cn);
        __builtin_amdgcn_sched_barrier(0);
        write_state(L.Hs + ((c + 1) & 1) * kP * HS);
        lds_barrier();
    }

    float* fin = (c1 == span.nch && prm.final_state) ? prm.final_state + unit * N * kP : nullptr;
    if (fin) {
#pragma unroll
        for (int jn = 0; jn < NBW; ++jn)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int n = 16 * (SW + 4 * jn) + 4 * lg;
                float* dst = fin + n * kP + 16 * pb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * kP] = hs[jn][pb][i];
            }
    }
}

// The work index of workgroup bid of a packed batch's walk: the (sequence, head) items in
// seq_order's order (longest first), one per workgroup.  Workgroups go to the 8 XCDs in turn, so
// every XCD gets every eighth item: a like share of each sequence's heads, and within an XCD the
// longest items start first.  (Dealing whole sequences to the XCDs kept a sequence's heads on one
// L2 but gave the XCD holding the longest sequence of each eight the most work.)  -1 past the
// last item.
__device__ __forceinline__ int64_t packed_work_index(const Walk2Params& prm, int64_t bid) {
    const int64_t r = bid / prm.nheads;
    if (r >= prm.batch) return -1;
    return (int64_t)prm.seq_order[r] * prm.nheads + bid % prm.nheads;
}

// DT: with log2 of an input scale per token (prm.lg_t, the discretisation front-end's Delta):
// the input side of every factor carries it, so the input term is Delta_s B_s x_s^T.
// PK: a packed batch walked as one sequence, with the recurrence restarted at every token
// prm.tok_flags marks (above).
// XS: x read with streaming loads (the host's choice for walks whose x is larger than the caches).
template <int N, int Q, bool DT, bool PK, bool XS>
__global__ void __launch_bounds__(kWalkThreads) walk_fast_kernel(Walk2Params prm) {
    const int64_t work = prm.seq_order ? packed_work_index(prm, blockIdx.x)
                                       : xcd_work_index(blockIdx.x, prm.per_xcd, prm.nseg * prm.batch * prm.nheads);
    if (work < 0) return;
    const WalkSpan span = walk_span(prm, work, Q);
    if (span.c1 <= span.c0) {
        // an empty packed sequence: its final state is its initial state
        if (prm.final_state)
            for (int i = threadIdx.x; i < N * kP; i += kWalkThreads)
                prm.final_state[span.unit * N * kP + i] = prm.init ? prm.init[span.unit * N * kP + i] : 0.f;
        return;
    }
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    extern __shared__ __align__(16) unsigned char smem[];
    const WalkLds<N, Q> L(smem);
    switch (wave) {
        case 0: walk_output_role<N, Q, 0, DT, PK>(prm, L, span, lane); break;
        case 1: walk_output_role<N, Q, 1, DT, PK>(prm, L, span, lane); break;
        case 2: walk_output_role<N, Q, 2, DT, PK>(prm, L, span, lane); break;
        case 3: walk_output_role<N, Q, 3, DT, PK>(prm, L, span, lane); break;
        case 4: walk_state_role<N, Q, 0, DT, PK>(prm, L, span, lane); break;
        case 5: walk_state_role<N, Q, 1, DT, PK>(prm, L, span, lane); break;
        case 6: walk_state_role<N, Q, 2, DT, PK>(prm, L, span, lane); break;
        case 7: walk_state_role<N, Q, 3, DT, PK>(prm, L, span, lane); break;
        case 8: walk_helper_role<N, Q, 0, DT, PK, XS>(prm, L, span, lane); break;
        case 9: walk_helper_role<N, Q, 1, DT, PK, XS>(prm, L, span, lane); break;
        case 10: walk_helper_role<N, Q, 2, DT, PK, XS>(prm, L, span, lane); break;
        default: walk_helper_role<N, Q, 3, DT, PK, XS>(prm, L, span, lane); break;
    }
}

// log2 weight below which exp2 is 0 in fp32 whatever its last-bit error (the smallest denormal
// is 2^-149)
constexpr float kVanish2 = -160.f;
// log2 of the largest input scale (the front-end's Delta) the early exit below allows for: with
// one, a token weighs at most 2^(decay + 64)
constexpr float kLog2ScaleMax = 64.f;

// seg_state_kernel: the state-only pass of a segmented walk.  One workgroup of four waves per
// (segment, batch, head) forms the segment's local state (its final state from a zero start) as
// one sum over the segment's chunks,
//   H_seg = sum_c B_c^T (W_c o X_c),   W_s = exp(decay from token s to the segment's end),
// which equals the chunk recurrence H_k = exp(cum_last) H_{k-1} + B^T (w o X) unrolled.  The
// chunks are taken last to first, so the decay from a chunk's end to the segment's end is the
// running sum of the chunks already done, W_s <= 1, and the state registers are only ever
// accumulated into.  Wave v holds rows 16 (v + 4 j) .. + 15 of the N x P state (a quarter of the
// MFMAs) and stages a quarter of the chunk's rows of W o x into a double-buffered LDS tile, which
// every wave reads back as MFMA operands contracting over tokens; one barrier per chunk, so the
// next chunk is staged while this one's MFMAs run.  Every wave scans the whole chunk's log a (the
// same values, so the same decays and the same early exit in each).  Once the weights of all
// tokens left are below 2^-160, where exp2 is 0 in fp32, the rest of the segment would add exact
// zeros: the pass then only sums the remaining chunks' decay, and the result is the same bit for
// bit.  (One wave holding the whole state took 20 us at the 32-sequence packed batch of the
// Mamba-2 layer's tokens, 128 MFMAs per chunk on one SIMD.)
constexpr int kSegWaves = 4;
template <int N, int Q>
struct SegStateShape {
    static constexpr int NBK = N / 16, NBW = NBK / kSegWaves, KS = Q / 32, PB = kP / 16, LA = Q / 64;
    static constexpr int QW = Q / kSegWaves, XR = QW * kP / 8 / kWave;  // rows and 16-byte pieces per wave
    static_assert(NBW >= 1 && XR >= 1, "segment state shape");
    // two W o x tiles [Q][kXStr] bf16, then W [Q] fp32
    static constexpr size_t lds_bytes = (size_t)2 * Q * kXStr * 2 + (size_t)Q * 4;
};

// PK: a packed batch walked as one sequence: a token marked in prm.tok_flags begins a new stretch
// of the recurrence, so every token before the segment's last marked token weighs 0, and the
// segment's decay is kRestart2 when it holds one (the walk's chain then restarts there).
template <int N, int Q, bool DT, bool PK>
__global__ void __launch_bounds__(kSegWaves * kWave) seg_state_kernel(Walk2Params prm) {
    using S = SegStateShape<N, Q>;
    constexpr int NBW = S::NBW, KS = S::KS, PB = S::PB, LA = S::LA, QW = S::QW, XR = S::XR;
    constexpr int NBK = S::NBK;
    const int64_t units = prm.batch * prm.nheads;
    const int64_t work = xcd_work_index(blockIdx.x, prm.per_xcd, (prm.nseg - 1) * units);
    if (work < 0) return;
    const WalkSpan span = walk_span(prm, work, Q);
    const int lane = threadIdx.x % kWave, wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t b = span.b, h = span.h, g = span.g, unit = span.unit;
    const int c0 = span.c0, c1 = span.c1;
    const int64_t H = prm.nheads, G = prm.ngroups;
    const int nchunks = prm.nchunks;
    const uint32_t x_row = (uint32_t)(H * kP * 2);
    const float* la0 = prm.la_t + unit * (int64_t)nchunks * Q;
    const float* lg0 = DT ? prm.lg_t + unit * (int64_t)nchunks * Q : nullptr;
    __bf16* xg = const_cast<__bf16*>(static_cast<const __bf16*>(prm.x));
    const __bf16* bt0 = prm.bt + (b * G + g) * (int64_t)nchunks * NBK * KS * 512;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Xw = reinterpret_cast<__bf16*>(smem);  // [2][Q][kXStr]
    // W of this wave's rows, permuted so that the XR rows a lane stages (r0 + lane / 8 + 8 m) are
    // contiguous
    float* wv_all = reinterpret_cast<float*>(smem + (size_t)2 * Q * kXStr * 2);
    float* wvw = wv_all + wv * QW;
    const int r0 = wv * QW;  // this wave's first row of a chunk
    auto chunk_len = [&](int c) { return (int)min((int64_t)Q, span.len - (int64_t)c * Q); };
    // staging piece m of this lane: row r0 + lane / 8 + 8 m, bytes 16 (lane % 8) of it
    const uint32_t xoff = (uint32_t)(r0 + lane / 8) * x_row + 16 * (lane % 8);

    float la[LA];
    float lgs[DT ? LA : 1];  // (DT) log2 of the input scale of the same tokens
    int flg[PK ? LA : 1];    // (PK) the token flags of the same tokens
    uint4 xs[XR];
    auto load_la = [&](int c) {
#pragma unroll
        for (int j = 0; j < LA; ++j) la[j] = la0[(int64_t)c * Q + lane * LA + j];
        if (DT)
#pragma unroll
            for (int j = 0; j < LA; ++j) lgs[j] = lg0[(int64_t)c * Q + lane * LA + j];
        if (PK)
#pragma unroll
            for (int j = 0; j < LA; ++j) flg[j] = prm.tok_flags[(int64_t)c * Q + lane * LA + j];
    };
    // this wave's x rows of the chunk through a buffer resource ending with it: rows past a short
    // chunk's end read as zeros
    auto load_x = [&](int c) {
        const __amdgpu_buffer_rsrc_t xr =
            buffer_rsrc(xg + ((span.row0 + (int64_t)c * Q) * H + h) * kP, (uint32_t)chunk_len(c) * x_row);
#pragma unroll
        for (int m = 0; m < XR; ++m) xs[m] = buffer_load16(xr, xoff + (uint32_t)(8 * m) * x_row);
    };
    // W o x of this wave's rows of chunk c into tile c & 1 (from la and xs of chunk c), with sfx2
    // the log2 decay from the chunk's end to the segment's end; returns the chunk's own log2 decay
    auto stage = [&](int c, float sfx2) -> float {
        const int len = chunk_len(c);
        float cum[LA], run = 0.f;
#pragma unroll
        for (int j = 0; j < LA; ++j) { run += (lane * LA + j < len) ? la[j] : 0.f; cum[j] = run; }
        const float incl = wave_inclusive_sum(run);
        const float excl = incl - run;
        float last2 = lane_value(incl, kWave - 1) * kLog2e;
        // (PK) the chunk's last marked token: the tokens before it weigh 0, and so does every
        // earlier chunk (the chunk's decay then stands for a restart)
        int knew = -1;
        if constexpr (PK) {
#pragma unroll
            for (int j = 0; j < LA; ++j)
                if (flg[j] != 0) knew = lane * LA + j;
            knew = wave_max(knew);
        }
        // (the lanes holding this wave's rows write their weights)
        if (lane * LA >= r0 && lane * LA < r0 + QW) {
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const int t = lane * LA + j, tl = t - r0;
                const float wt = fexp2(sfx2 + (last2 - (excl + cum[j]) * kLog2e) + (DT ? lgs[j] : 0.f));
                wvw[(tl % 8) * (QW / 8) + tl / 8] = (!PK || t >= knew) ? wt : 0.f;
            }
        }
        if (PK && knew >= 0) last2 = kRestart2;
        wave_lds_fence();
        // (row r0 + lane / 8 + 8 m sits at (lane / 8) XR + m: QW / 8 = XR)
        float w[XR];
#pragma unroll
        for (int m = 0; m < XR; ++m) w[m] = wvw[(lane / 8) * XR + m];
        __bf16* tile = Xw + (c & 1) * Q * kXStr;
#pragma unroll
        for (int m = 0; m < XR; ++m) {
            const bf16x8 rv = as_bf16x8(xs[m]);
            bf16x8 sv;
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[j] = (__bf16)((float)rv[j] * w[m]);
            *reinterpret_cast<bf16x8*>(tile + (r0 + lane / 8 + 8 * m) * kXStr + 8 * (lane % 8)) = sv;
        }
        return last2;
    };

    f32x4 hs[NBW][PB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) hs[j][pb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunks last to first; sfx2 = log2 decay from the end of the chunk being staged to the
    // segment's end
    load_la(c1 - 1);
    load_x(c1 - 1);
    float sfx2 = stage(c1 - 1, 0.f);
    load_la(max(c1 - 2, c0));
    load_x(max(c1 - 2, c0));
    for (int c = c1 - 1; c >= c0; --c) {
        // chunk c staged by every wave; every wave done reading tile (c - 1) & 1 (chunk c + 1)
        __syncthreads();
        const void* bbase = bt0 + (int64_t)c * NBK * KS * 512;
        uint4 bt[NBW][KS];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int k = 0; k < KS; ++k) bt[j][k] = ldg16(bbase, 16 * lane + ((wv + kSegWaves * j) * KS + k) * 1024);
        const __bf16* tile = Xw + (c & 1) * Q * kXStr;
        bf16x8 xfa[KS][PB];
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) xfa[k][pb] = token_frag(tile, kXStr, 16 * pb, k, lane);
        // the chunk before into the other tile (the other waves may still read this one)
        const float bound2 = sfx2;  // every token before chunk c weighs at most 2^bound2
        if (c > c0) sfx2 += stage(c - 1, sfx2);
        load_la(max(c - 2, c0));
        load_x(max(c - 2, c0));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int k = 0; k < KS; ++k)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) hs[j][pb] = mfma_bf16(as_bf16x8(bt[j][k]), xfa[k][pb], hs[j][pb]);
        if (bound2 < kVanish2 - (DT ? kLog2ScaleMax : 0.f)) {
            // The weights of all earlier tokens are 0 in fp32 (exp2 of less than -160), so the
            // earlier chunks would add exact zeros: only their decay is still summed.  (PK: after
            // a restart the segment's decay stands for the restart whatever the earlier chunks
            // hold, so nothing is left to do.)  (Every wave takes this branch together.)
            if (PK && sfx2 <= 0.5f * kRestart2) break;
            for (int cc = c - 2; cc >= c0; --cc) {
                load_la(cc);
                const int len = chunk_len(cc);
                float run = 0.f;
#pragma unroll
                for (int j = 0; j < LA; ++j) run += (lane * LA + j < len) ? la[j] : 0.f;
                sfx2 += lane_value(wave_inclusive_sum(run), kWave - 1) * kLog2e;
            }
            break;
        }
    }

    const int64_t sidx = span.seg * units + unit;
    if (wv == 0 && lane == 0) prm.seg_decay[sidx] = sfx2;
    float* fin = prm.seg_state + sidx * N * kP;
    const int l16 = lane % 16, lg = lane / 16;
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            float* dst = fin + (16 * (wv + kSegWaves * j) + 4 * lg) * kP + 16 * pb + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i * kP] = hs[j][pb][i];
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

// Workspace layout of the fast path (byte offsets), for Q-token chunks.
struct FastLayout {
    int64_t nchunks, nblk, units;
    int nseg, seg_chunks;
    size_t pairs, bt, ct, la_t, lg_t, seg_state, seg_decay, order, flags, total;
};

// segments of a walk over `units` units of any length: at most this many
constexpr int seg_cap(int64_t units) { return units > 0 && units * 2 <= 256 ? (int)(kSegTarget / units) : 1; }

// (with_lg: log2 of the input scale head-major, laid out as la_t; varlen: a packed
// variable-length batch walked sequence by sequence, never segmented; packed_cap > 0: a packed
// batch walked as one sequence of seqlen tokens, batch 1, with every array sized for packed_cap
// tokens and the most segments any length gives, and the token flags at the end)
FastLayout fast_layout(int64_t batch, int64_t nheads, int64_t ngroups, int64_t seqlen, int N, int Q,
                       bool with_lg = false, bool varlen = false, int64_t packed_cap = 0) {
    FastLayout l;
    l.nchunks = (seqlen + Q - 1) / Q;
    l.nblk = batch * ngroups * l.nchunks;
    l.units = batch * nheads;
    // capacities: chunks per unit and segments
    const int64_t cap_chunks = packed_cap > 0 ? (packed_cap + Q - 1) / Q : l.nchunks;
    const int64_t cap_blk = batch * ngroups * cap_chunks;
    // One round of walk workgroups (see kSegTarget).
    if (varlen) {
        l.nseg = 1;
        l.seg_chunks = (int)(l.nchunks > 0 ? l.nchunks : 1);
    } else {
        l.nseg = walk_segments(l.units, l.nchunks, kSegTarget, &l.seg_chunks);
    }
    const int cap_seg = packed_cap > 0 ? (l.nseg > seg_cap(l.units) ? l.nseg : seg_cap(l.units)) : l.nseg;
    size_t off = 0;
    l.pairs = off; off += (size_t)cap_blk * n_pairs(Q / 16) * 1024;
    l.bt = off; off += (size_t)cap_blk * N * Q * 2;
    l.ct = off; off += (size_t)cap_blk * N * Q * 2;
    l.la_t = off; off += (size_t)l.units * cap_chunks * Q * 4;
    l.lg_t = off;
    if (with_lg) off += (size_t)l.units * cap_chunks * Q * 4;
    l.seg_state = l.seg_decay = off;
    if (cap_seg > 1) {
        l.seg_state = off; off += (size_t)cap_seg * l.units * N * kP * 4;
        l.seg_decay = off; off += ((size_t)cap_seg * l.units * 4 + 255) / 256 * 256;
    }
    // a packed batch of at most kOrderMax sequences: their order, longest first
    l.order = off;
    if (varlen && batch <= kOrderMax) off += ((size_t)batch * 4 + 255) / 256 * 256;
    // a packed batch walked as one sequence: the token flags, one int per token of whole chunks
    l.flags = off;
    if (packed_cap > 0) off += (size_t)cap_chunks * Q * 4;
    l.total = off;
    return l;
}

// The token flags of a packed batch walked as one sequence (Walk2Params::tok_flags), for the
// tokens of whole chunks (npad), when the batch has too many sequences for the prep kernel to
// mark them: one workgroup clears them, then marks every nonempty sequence's
// first token as a start, and as outside every sequence the tokens before the first offset, from
// the last offset on, and those past a sequence's first `bound` (the length bound every sequence is
// walked to).  Offsets are clamped into [0, total] as the sequence-by-sequence walk clamps them.
constexpr int kMarkThreads = 1024;
__global__ void __launch_bounds__(kMarkThreads) mark_tokens_kernel(const int64_t* seq_off, int64_t nseq, int64_t total,
                                                                   int64_t bound, int* flags, int64_t npad) {
    const int tid = threadIdx.x;
    for (int64_t i = 4 * (int64_t)tid; i < npad; i += 4 * kMarkThreads)
        *reinterpret_cast<int4*>(flags + i) = int4{0, 0, 0, 0};
    __syncthreads();
    auto clampt = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > total ? total : v); };
    for (int64_t j = tid; j < nseq; j += kMarkThreads) {
        const int64_t s = clampt(seq_off[j]);
        int64_t e = clampt(seq_off[j + 1]);
        e = e < s ? s : e;
        if (e > s) atomicOr(flags + s, kFlagStart);
        for (int64_t t = s + bound; t < e; ++t) atomicOr(flags + t, kFlagStart | kFlagDead);
    }
    const int64_t lo = clampt(seq_off[0]), hi = clampt(seq_off[nseq]);
    for (int64_t t = tid; t < lo; t += kMarkThreads) atomicOr(flags + t, kFlagStart | kFlagDead);
    for (int64_t t = hi + tid; t < total; t += kMarkThreads) atomicOr(flags + t, kFlagStart | kFlagDead);
}

// packed_cap > 0: fl describes a packed batch walked as one sequence (batch 1, seqlen = its tokens,
// no offsets), whose token flags the workspace holds (fast_layout with this packed_cap); with
// mark_off non-null the prep kernel writes them from the batch's mark_nseq + 1 offsets (at most
// kMarkLdsMax) and its length bound, else a marking launch already has
template <int N, int Q, bool DT, bool PK>
int launch_fast_core(const ForwardLaunch& fl, hipStream_t stream, int64_t packed_cap, const int64_t* mark_off = nullptr,
                     int64_t mark_nseq = 0, int64_t mark_bound = 0) {
    static_assert(WalkShape<N, Q>::lds_bytes <= kMaxLds, "walk LDS budget");
    static bool prep_attr[64] = {}, walk_attr[64] = {}, walk_xs_attr[64] = {};
    const bool with_lg = fl.dt && fl.scale_input;
    const FastLayout lay =
        fast_layout(fl.batch, fl.nheads, fl.ngroups, fl.seqlen, N, Q, with_lg, fl.seq_off != nullptr, packed_cap);
    char* ws = reinterpret_cast<char*>(fl.scores);
    __bf16* pairs = reinterpret_cast<__bf16*>(ws + lay.pairs);
    __bf16* bt = reinterpret_cast<__bf16*>(ws + lay.bt);
    __bf16* ct = reinterpret_cast<__bf16*>(ws + lay.ct);
    float* la_t = reinterpret_cast<float*>(ws + lay.la_t);
    const int nch = (int)lay.nchunks;
    float* lg_t = with_lg ? reinterpret_cast<float*>(ws + lay.lg_t) : nullptr;
    PrepParams pp{fl.Bm, fl.Cm, fl.log_a, pairs, bt, ct, la_t, fl.dt, fl.dt_bias, fl.A_log, lg_t,
                  fl.seqlen, fl.nheads, fl.ngroups, nch, lay.nblk, 0, fl.seq_off, fl.total, nullptr};
    if (!allow_full_lds(reinterpret_cast<const void*>(&prep_kernel<N, Q>), prep_attr)) return -1;
    // x read with streaming loads when the walk's x alone is larger than the 256 MB last-level
    // cache (packed batches excepted): then keeping x would only evict the group-shared operands
    // that every head of a group reads again.  (Gqa decode workload, 268 MB of x: walk 196 -> 179
    // us; long sequence 268 MB: forward 256-263 -> 249-251 us; at the Mamba-2 layer shape, 50 MB of
    // x, the streaming loads cost 2-3 us per forward.)
    const bool xs = !PK && (double)fl.batch * (double)fl.seqlen * (double)fl.nheads * kP * 2.0 > kXStreamBytes;
    const auto walk = xs ? walk_fast_kernel<N, Q, DT, PK, !PK> : walk_fast_kernel<N, Q, DT, PK, false>;
    if (!allow_full_lds(reinterpret_cast<const void*>(walk), xs ? walk_xs_attr : walk_attr)) return -1;
    int k = fl.first_launch;
    size_t plds = prep_lds<N, Q>();
    const size_t slds = SegStateShape<N, Q>::lds_bytes, wlds = WalkShape<N, Q>::lds_bytes;
    if (PK && mark_off) {
        if (mark_nseq < 0 || mark_nseq + 1 > kMarkLdsMax) return -1;
        pp.mark_off = mark_off;
        pp.mark_nseq = mark_nseq;
        pp.mark_bound = mark_bound;
        pp.flags = reinterpret_cast<int*>(ws + lay.flags);
        plds += ((size_t)(mark_nseq + 1) * 4 + 15) / 16 * 16;
        static_assert(prep_lds<N, Q>() + (size_t)kMarkLdsMax * 4 <= kMaxLds, "offsets in the prep kernel's LDS");
    }
    const unsigned pthreads = PrepShape<N, Q>::THREADS;
    // split each block over two workgroups when even then they fit on the CUs at once
    pp.split = 2 * lay.nblk <= kPrepSplitMax ? 1 : 0;
    const unsigned pgrid = pp.split ? (unsigned)((lay.nblk + 7) / 8 * 16) : (unsigned)lay.nblk;
    // (a packed batch: the sequences ranked longest first, for the walk's workgroup order, by one
    // more prep workgroup, whose LDS holds every length)
    static_assert(prep_lds<N, Q>() >= (size_t)kOrderMax * 4, "sequence lengths in the prep kernel's LDS");
    int* order = (fl.seq_off && fl.batch <= kOrderMax) ? reinterpret_cast<int*>(ws + lay.order) : nullptr;
    pp.order = order;
    const unsigned rgrid = order ? (unsigned)ranking_groups<PrepShape<N, Q>::THREADS>(fl.batch) : 0u;
    if (!launch_k(fl, k, prep_kernel<N, Q>, dim3(pgrid + rgrid), dim3(pthreads), plds, stream, pp)) return -1;

    const int64_t work = lay.nseg * lay.units;
    // (ordered packed walk: one workgroup per (sequence, head), dealt to the XCDs in turn)
    const int64_t per_xcd = order ? (fl.batch * fl.nheads + 7) / 8 : (work + 7) / 8;
    Walk2Params wp{fl.x, la_t, lg_t, ct, fl.D, pairs, bt, fl.init, fl.y, fl.final_state,
                   fl.batch, fl.seqlen, fl.nheads, fl.ngroups, nch, per_xcd,
                   lay.seg_chunks, lay.nseg, reinterpret_cast<float*>(ws + lay.seg_state),
                   reinterpret_cast<float*>(ws + lay.seg_decay), fl.seq_off, fl.total, order,
                   PK ? reinterpret_cast<const int*>(ws + lay.flags) : nullptr};
    if (lay.nseg > 1) {
        // (the last segment's local state is never needed: only segments 0 .. nseg-2)
        const int64_t state_work = (lay.nseg - 1) * lay.units;
        Walk2Params sp = wp;
        sp.per_xcd = (state_work + 7) / 8;
        if (!launch_k(fl, k, seg_state_kernel<N, Q, DT, PK>, dim3((unsigned)(8 * sp.per_xcd)), dim3(kSegWaves * kWave), slds,
                      stream, sp))
            return -1;
        // (each walk workgroup chains the segment states into its own start state)
    }
    return launch_k(fl, k, walk, dim3((unsigned)(8 * per_xcd)), dim3(kWalkThreads), wlds,
                    stream, wp)
               ? 0
               : -1;
}

// A packed batch with no initial or final states requested can be walked as one sequence of all
// its tokens (segmented like a long batched sequence), with the recurrence restarted at every
// sequence's first token: the work is then proportional to tokens, not to sequences, and long
// sequences are split over several workgroups.  (Per-sequence states need the sequence-by-sequence
// walk: a sequence that ends or starts inside a chunk has its state nowhere else.)  The host knows
// the sequence count, the token count and the length bound, and takes the form with the shorter
// estimated walk, in chunk periods: sequence by sequence at least the longest sequence's chunks
// and the chunks of all (sequence, head) walks spread over 256 CUs; as one sequence the chunks of
// one segment, plus its state pass (~0.35 of them), the segment-state launch and the marking in
// prep (~2).  (Mamba-2 layer tokens, log-normal lengths: 8 / 128 / 1024 sequences 66.5 / 61.5 /
// 58.9 us as one sequence, 92 / 113 / 545 us sequence by sequence; 32 sequences 60.8 us sequence
// by sequence, 69 us as one with the marking in a launch of its own.)
template <int Q>
bool packed_as_one(const ForwardLaunch& fl) {
    if (!fl.seq_off || fl.init || fl.final_state || fl.total <= 0) return false;
    const int64_t nch = (fl.total + Q - 1) / Q;
    int per = 1;
    walk_segments(fl.nheads, nch, kSegTarget, &per);
    const double as_one = 1.35 * per + 2.0;
    const double longest = (double)((fl.seqlen + Q - 1) / Q);
    const double spread = std::ceil((double)(nch + fl.batch) * (double)fl.nheads / 256.0);
    return as_one < (longest > spread ? longest : spread);
}

template <int N, int Q, bool DT>
int launch_fast_t(const ForwardLaunch& fl, hipStream_t stream) {
    if (!packed_as_one<Q>(fl)) return launch_fast_core<N, Q, DT, false>(fl, stream, 0);
    ForwardLaunch one = fl;
    one.batch = 1;
    one.seqlen = fl.total;
    one.nchunks = (int)((fl.total + Q - 1) / Q);
    one.seq_off = nullptr;
    // arrays sized for the most tokens the batch can hold, as the workspace query sizes them
    const int64_t cap = fl.batch * fl.seqlen;
    const bool with_lg = fl.dt && fl.scale_input;
    const FastLayout lay = fast_layout(1, fl.nheads, fl.ngroups, one.seqlen, N, Q, with_lg, false, cap);
    // (up to kMarkLdsMax - 1 sequences the prep kernel marks the tokens; more take a launch)
    if (fl.batch + 1 <= kMarkLdsMax && fl.total <= INT32_MAX)
        return launch_fast_core<N, Q, DT, true>(one, stream, cap, fl.seq_off, fl.batch, fl.seqlen);
    int* flags = reinterpret_cast<int*>(reinterpret_cast<char*>(fl.scores) + lay.flags);
    int k = fl.first_launch;
    if (!launch_k(fl, k, mark_tokens_kernel, dim3(1), dim3(kMarkThreads), 0, stream, fl.seq_off, fl.batch, fl.total,
                  fl.seqlen, flags, (int64_t)lay.nchunks * Q))
        return -1;
    one.first_launch = k;
    return launch_fast_core<N, Q, DT, true>(one, stream, cap);
}

}  // namespace

// Chunks of 256 tokens run as two 128-token chunks: the same operator, evaluated with the
// state carried at every 128th token instead of every 256th.
int fast_chunk(int chunk) { return chunk > 128 ? 128 : chunk; }

bool fast_path_applies(int dtype, int decay, int N, int P, int chunk, int64_t nheads, int64_t ngroups) {
    // byte offsets inside one chunk (chunk rows of x, y, B, C) must fit in 32 bits, and the prep
    // kernel moves the log a of at most kPrepLa * 4 * kPrepThreads / chunk heads per group
    const int q = fast_chunk(chunk);
    const bool offsets_fit = (double)q * (double)(nheads * P + ngroups * N) * 2.0 < 2147483648.0;
    const bool heads_fit = ngroups > 0 && nheads / ngroups <= (int64_t)kPrepLa * 4 * kPrepMinThreads / q;
    return dtype == 1 && decay == 0 && P == kP && (N == 64 || N == 128) &&
           (chunk == 64 || chunk == 128 || chunk == 256) && offsets_fit && heads_fit;
}

size_t fast_workspace_bytes(int64_t batch, int64_t nheads, int64_t ngroups, int64_t seqlen, int N, int chunk,
                            bool with_lg, bool varlen) {
    const int Q = fast_chunk(chunk);
    const size_t own = fast_layout(batch, nheads, ngroups, seqlen, N, Q, with_lg, varlen).total;
    if (!varlen) return own;
    // (a packed batch may be walked as one sequence of up to batch * seqlen tokens)
    const int64_t cap = batch * seqlen;
    const size_t one = fast_layout(1, nheads, ngroups, cap, N, Q, with_lg, false, cap).total;
    return own > one ? own : one;
}

int launch_forward_fast(const ForwardLaunch& fl, hipStream_t stream) {
    const int N = (int)fl.dstate, Q = fast_chunk(fl.chunk);
    // (the scaled-input form only when the input scale exists: log a from dt alone needs nothing
    // in the walk)
    const bool dt = fl.dt && fl.scale_input;
    if (N == 64 && Q == 64) return dt ? launch_fast_t<64, 64, true>(fl, stream) : launch_fast_t<64, 64, false>(fl, stream);
    if (N == 64 && Q == 128)
        return dt ? launch_fast_t<64, 128, true>(fl, stream) : launch_fast_t<64, 128, false>(fl, stream);
    if (N == 128 && Q == 64)
        return dt ? launch_fast_t<128, 64, true>(fl, stream) : launch_fast_t<128, 64, false>(fl, stream);
    if (N == 128 && Q == 128)
        return dt ? launch_fast_t<128, 128, true>(fl, stream) : launch_fast_t<128, 128, false>(fl, stream);
    return -2;
}

// Chains the segments' local states, one thread per state element (n, p) of one unit:
//   seg_init[s] = exp2(decay[s-1]) o seg_init[s-1] + seg_state[s-1],  seg_init[0] = init (or 0),
// with decay one log2 value per (segment, unit) (per_n = 0) or per (segment, unit, n) (per_n = 1).
// States are [segment][unit][N][P] fp32.  (The diagonal walk uses it; the scalar walk chains the
// states in each workgroup.)
__global__ void __launch_bounds__(kThreads) seg_prefix_kernel(const float* init, float* seg_init,
                                                              const float* seg_state, const float* seg_decay,
                                                              int64_t units, int N, int P, int nseg, int per_n) {
    const int64_t epu = (int64_t)N * P;
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= units * epu) return;
    const int64_t unit = e / epu;
    const int n = (int)((e % epu) / P);
    const int64_t dstride = per_n ? N : 1;
    const int64_t didx = unit * dstride + (per_n ? n : 0);
    float hcur = init ? init[e] : 0.f;
    for (int s = 0; s < nseg; ++s) {
        seg_init[s * units * epu + e] = hcur;
        if (s + 1 < nseg)
            hcur = exp2f(seg_decay[s * units * dstride + didx]) * hcur + seg_state[s * units * epu + e];
    }
}

int launch_seg_prefix(const ForwardLaunch& fl, int& k, const float* init, float* seg_init, const float* seg_state,
                      const float* seg_decay, int64_t units, int N, int P, int nseg, int per_n, hipStream_t stream) {
    const int64_t total = units * N * P;
    return launch_k(fl, k, seg_prefix_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                    stream, init, seg_init, seg_state, seg_decay, units, N, P, nseg, per_n)
               ? 0
               : -1;
}

}  // namespace ssd
