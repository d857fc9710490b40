// Device-side helpers shared by the SSD kernels: vector types, MFMA wrappers, 16-byte
// memory moves and a block-wide inclusive scan.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Per element type: MFMA K-depth handled by one "K block" and elements per 16 bytes.
//   bf16: one v_mfma_f32_16x16x32_bf16 per K block of 32 (lane group g holds k = 8g..8g+7)
//   fp32: four v_mfma_f32_16x16x4_f32 per K block of 16 (MFMA i: lane group g holds
//         k = 4g+i, so a lane's 16-byte read of k = 4g..4g+3 feeds all four)
template <typename T> struct Traits;
template <> struct Traits<__bf16> {
    static constexpr int kKBlock = 32;
    static constexpr int kVec = 8;   // elements per 16 bytes
    static constexpr int kPad = 8;   // LDS row padding in elements (16 bytes)
};
template <> struct Traits<float> {
    static constexpr int kKBlock = 16;
    static constexpr int kVec = 4;
    static constexpr int kPad = 4;
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x4 as_f32x4(uint4 v) { return __builtin_bit_cast(f32x4, v); }

__device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

// Four consecutive elements as one 8-byte (bf16) or 16-byte (fp32) store.
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// The step size of the discretisation front-end: softplus(v) = log(1 + e^v), written as
// max(v, 0) + log(1 + e^-|v|) so that no intermediate overflows.
__device__ __forceinline__ float softplusf(float v) { return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v))); }
__device__ __forceinline__ double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }
// log2 softplus(v).  Below v = -20, softplus(v) = e^v (1 - e^v / 2 + ...), so log2 of it is
// v log2(e) to within 2e-9; that form stays exact where softplus(v) itself underflows.
__device__ __forceinline__ float log2_softplusf(float v) {
    return v < -20.f ? v * 1.4426950408889634f : log2f(softplusf(v));
}

// softplus on the hardware exp2 and log2 units (v_exp_f32, v_log_f32), for the bf16 paths'
// front-end.  With e = e^-|v| in (0, 1], log(1 + e) is the series e - e^2/2 + e^3/3 - e^4/4
// below e = 2^-6 (truncation under e^5/5) and log2(1 + e) ln 2 above, where rounding 1 + e
// costs at most 2^-18 of e: a relative error of a few 1e-6 in all.  Below v = -87 (e under the
// normal range) the result is max(v, 0) = 0.
__device__ __forceinline__ float softplus_hw(float v) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(v) * 1.4426950408889634f);
    const float series = e * (1.f - e * (0.5f - e * (0.33333334f - 0.25f * e)));
    const float l = e < 0.015625f ? series : __builtin_amdgcn_logf(1.f + e) * 0.6931471805599453f;
    return fmaxf(v, 0.f) + l;
}
// log2 of softplus(v) = sp (from softplus_hw): v log2(e) below v = -20, as in log2_softplusf.
__device__ __forceinline__ float log2_softplus_hw(float v, float sp) {
    return v < -20.f ? v * 1.4426950408889634f : __builtin_amdgcn_logf(sp);
}

// Barrier that orders LDS accesses only: global loads, stores and atomics issued before it stay in
// flight (a kernel whose threads share data only through LDS needs no more).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block-wide inclusive scan of one value per thread (kThreads threads).  `scratch` holds
// kWaves values of type V in LDS.  Contains two __syncthreads().
template <typename V>
__device__ __forceinline__ V block_inclusive_scan(V v, V* scratch) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        V o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) scratch[wave] = v;
    __syncthreads();
    V prefix = 0;
    for (int w = 0; w < wave; ++w) prefix += scratch[w];
    __syncthreads();
    return v + prefix;
}

// Maps a launch index to a work index so that each of the 8 XCDs (which receive workgroups
// round-robin) gets one contiguous range of work: neighbouring heads of one (batch, group)
// then share that XCD's L2.  Returns -1 for padding workgroups.
// The rows of sequence b.  Batched layout (seq_off null): tokens b * seqlen .. + seqlen of the
// [batch][seqlen] token axis.  Packed variable-length batch: tokens seq_off[b] .. seq_off[b+1] of the
// packed axis of `total` tokens, clamped into [0, total] and to at most seqlen tokens, so that any
// offsets keep every access inside the tensors and the workspace.
struct SeqSpan {
    int64_t row0, len;
};
__device__ __forceinline__ SeqSpan seq_span(const int64_t* seq_off, int64_t b, int64_t seqlen, int64_t total) {
    if (!seq_off) return SeqSpan{b * seqlen, seqlen};
    int64_t s = seq_off[b], e = seq_off[b + 1];
    s = s < 0 ? 0 : (s > total ? total : s);
    e = e < s ? s : (e > total ? total : e);
    return SeqSpan{s, e - s < seqlen ? e - s : seqlen};
}

__device__ __forceinline__ int64_t xcd_work_index(int64_t bid, int64_t per_xcd, int64_t total) {
    const int64_t w = (bid % 8) * per_xcd + bid / 8;
    return w < total ? w : -1;
}

}  // namespace ssd
