// Device-side building blocks shared by the gfx950 kernels of the MoE decode
// layer: element decoders, wavefront reductions and the per-workgroup
// expert-sorted work queue.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kWave = 64;
constexpr int kMaxTokens = 16;
constexpr int kMaxSlots = 16;
constexpr int kMaxPairs = kMaxTokens * kMaxSlots;
constexpr int kMaxExperts = 1025;  // routed + shared
constexpr int kBitmapWords = (kMaxExperts + 31) / 32;

enum { WFMT_MXFP4 = 1, WFMT_FP8_B128 = 2 };

// ---- element formats -------------------------------------------------------------------

// E8M0 block exponent -> fp32 2^(s-127); 0 -> 2^-127 (subnormal); 255 -> NaN.  Branch-free
// (selects), so it can sit in a load/compute pipeline without splitting it.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7FC00000u : bits;
  return __uint_as_float(bits);
}

// Four FP8 E4M3FN codes in one dword -> two bf16 pairs (exact: E4M3 fits bf16).
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}

// Eight E2M1 codes in one dword (element 2j in the low nibble of byte j) -> four bf16 pairs.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t w, bf16x2 (&o)[4]) {
  o[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  o[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  o[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  o[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
}

// Two FP8 codes (low or high half of the dword) -> two fp32.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
}

// Two E2M1 codes (byte SEL of the dword) -> two fp32.
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Opaque to the optimizer: the value may have changed.  Used inside per-token loops so that
// the decode of a weight chunk is redone per token instead of being hoisted out of the loop
// with every decoded value kept live (which would cost far more registers than it saves).
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// 16-byte streaming load (weights are read once per call: non-temporal hint).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---- wavefront reductions ----------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- expert-sorted work queue ------------------------------------------------------------
// Every workgroup rebuilds, from the M*S routing ids, the ascending list of distinct active
// experts and picks entry `q`; it then gathers that expert's (token, slot) pairs in pair
// order p = t*S + j.  Ids outside [0, n_experts) are ignored and reported through `invalid`.
struct QueueLds {
  int32_t ids[kMaxPairs];
  uint32_t bitmap[kBitmapWords];
  int32_t wave_count[16];
  int32_t expert;
  int32_t n_active;
  int32_t n_pairs;      // pairs of `expert`
  int32_t invalid;
  int16_t pairs[kMaxPairs];
};

// Returns the expert of queue entry q (or -1 when q >= number of active experts).
// Must be called by every thread of the workgroup (contains barriers).
__device__ int build_queue(QueueLds& Q, const int32_t* __restrict__ topk_ids, int n_pairs,
                           int n_experts, int q) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int i = tid; i < kBitmapWords; i += nthr) Q.bitmap[i] = 0u;
  if (tid == 0) Q.invalid = 0;
  __syncthreads();
  for (int i = tid; i < n_pairs; i += nthr) {
    const int e = topk_ids[i];
    Q.ids[i] = e;
    if (e >= 0 && e < n_experts)
      atomicOr(&Q.bitmap[e >> 5], 1u << (e & 31));
    else
      Q.invalid = 1;
  }
  __syncthreads();
  if (tid == 0) {
    int count = 0, found = -1;
    const int words = (n_experts + 31) >> 5;
    for (int w = 0; w < words; ++w) {
      uint32_t bits = Q.bitmap[w];
      const int pc = __popc(bits);
      if (found < 0 && q < count + pc) {
        int r = q - count;
        while (r-- > 0) bits &= bits - 1;  // drop the lowest set bits before the target
        found = (w << 5) + __builtin_ctz(bits);
      }
      count += pc;
    }
    Q.expert = found;
    Q.n_active = count;
    Q.n_pairs = 0;
  }
  __syncthreads();
  const int e = Q.expert;
  if (e < 0) return -1;
  // Ordered compaction of the pairs that selected e (ballot per wave, then wave offsets).
  const int wave = tid / kWave, lane = tid % kWave, nwaves = nthr / kWave;
  for (int base = 0; base < n_pairs; base += nthr) {
    const int i = base + tid;
    const bool hit = (i < n_pairs) && (Q.ids[i] == e);
    const uint64_t mask = __ballot(hit);
    if (lane == 0) Q.wave_count[wave] = __popcll(mask);
    __syncthreads();
    int offset = (base == 0) ? 0 : Q.n_pairs;
    for (int w = 0; w < wave; ++w) offset += Q.wave_count[w];
    if (hit) Q.pairs[offset + __popcll(mask & ((1ull << lane) - 1ull))] = (int16_t)i;
    __syncthreads();
    if (tid == 0) {
      int total = (base == 0) ? 0 : Q.n_pairs;
      for (int w = 0; w < nwaves; ++w) total += Q.wave_count[w];
      Q.n_pairs = total;
    }
    __syncthreads();
  }
  return e;
}

}  // namespace moe
