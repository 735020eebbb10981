// Live FP8 activation quantization of the W8A8 expert FFN.
//   d9249.github.io "glm-5-2-b300-kernel-mtp-serving", table under "what it solves" and idea 1:
//   the activations are quantized to FP8 inside the expert GEMM, where the work overlaps the
//   weight stream, rather than in a pass of their own; idea 3: the quantization changes the
//   model's outputs, a fidelity cost to be measured.
// Per 128 consecutive values of one token's activation row (the K extent of one weight scale
// block): s = fp32(amax/448), 1 for an all-zero block, NaN for a block holding a non-finite
// value; each value becomes the E4M3 value nearest fp32(v/s) (ties to even, saturating at 448).
// The kernels keep those values exactly (E4M3 fits bf16 and fp32), so their chunk dot products
// run unchanged, and fold s into the chunk's weight scale.  A block is held by G consecutive
// lanes, whose group maximum gives amax.
//
// Arithmetic per value: the quotient fp32(v/s) from a reciprocal and one residual correction,
// then the hardware's E4M3 conversion (round to nearest even) and its exact decode.
#pragma once
#include "moe_device.h"

namespace moe {
namespace {

template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) {
    const uint32_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// Block scale from the block's largest |v| as fp32 bits (non-finite inputs compare above
// every finite one).
__device__ __forceinline__ float act_scale(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return __builtin_nanf("");
  return amax_bits == 0 ? 1.0f : __fdiv_rn(__uint_as_float(amax_bits), 448.0f);
}

// The division of one block by its scale s, sign of v kept (also for -0).  With r = fp32(1/s)
// (correctly rounded), the product q = fp32(v*r) is within one ulp of v/s, its residual
// fma(-q, s, v) is exact, and fp32(q + residual*r) is the correctly rounded quotient
// (Markstein's theorem), provided the residual stays in fp32's normal range.  That holds for
// every v whose quotient can round to a nonzero code (|v/s| >= 2^-11) once s >= 2^-80.
// Smaller scales take the full division, clamped to +-448 as the conversion's saturation: a
// scale that rounded to zero or lost precision in fp32's subnormal range can give |v/s| > 448
// or 0/0, and every code then dequantizes to code * 0 = 0 or to a saturated 448 * s alike.
struct ActDiv {
  float s, r;
  bool full;
  __device__ explicit ActDiv(float scale)
      : s(scale), r(__frcp_rn(scale)), full(scale < 0x1p-80f) {}
  __device__ float operator()(float v) const {
    float t;
    if (full) {
      t = fminf(fmaxf(__fdiv_rn(v, s), -448.0f), 448.0f);
    } else {
      const float q = v * r;
      t = __builtin_fmaf(__builtin_fmaf(-q, s, v), r, q);
    }
    return __builtin_copysignf(t, v);
  }
};

// Four quotients -> one dword of E4M3 codes (byte i = value i), round to nearest even, sign
// kept, |t| <= 448 * (1 + 2^-23) here so nothing overflows.
__device__ __forceinline__ uint32_t e4m3x4_rne(float t0, float t1, float t2, float t3) {
  uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t2, t3, (int)c, true);
}

// A lane's bf16 activation pairs (NW words, NW even), quantized in place to the bf16 values of
// their codes; returns the block scale.
template <int G, int NW>
__device__ __forceinline__ float act_quant_bf16(uint32_t (&w)[NW]) {
  static_assert(NW % 2 == 0, "four values per code dword");
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
    amax = lo > amax ? lo : amax;
    amax = hi > amax ? hi : amax;
  }
  const float s = act_scale(group_max_u32<G>(amax) << 16);
  const ActDiv div(s);
#pragma unroll
  for (int j = 0; j < NW; j += 2) {
    const uint32_t c = e4m3x4_rne(div(__uint_as_float(w[j] << 16)),
                                  div(__uint_as_float(w[j] & 0xFFFF0000u)),
                                  div(__uint_as_float(w[j + 1] << 16)),
                                  div(__uint_as_float(w[j + 1] & 0xFFFF0000u)));
    bf16x2 lo, hi;
    fp8x4_to_bf16(c, lo, hi);
    w[j] = __builtin_bit_cast(uint32_t, lo);
    w[j + 1] = __builtin_bit_cast(uint32_t, hi);
  }
  return s;
}

// A lane's fp32 activations (N values, N a multiple of 4), quantized in place; returns the
// block scale.
template <int G, int N>
__device__ __forceinline__ float act_quant_f32(float (&v)[N]) {
  static_assert(N % 4 == 0, "four values per code dword");
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t b = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    amax = b > amax ? b : amax;
  }
  const float s = act_scale(group_max_u32<G>(amax));
  const ActDiv div(s);
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const uint32_t c = e4m3x4_rne(div(v[i]), div(v[i + 1]), div(v[i + 2]), div(v[i + 3]));
    const f32x2 lo = fp8x2_to_f32<false>(c), hi = fp8x2_to_f32<true>(c);
    v[i] = lo.x;
    v[i + 1] = lo.y;
    v[i + 2] = hi.x;
    v[i + 3] = hi.y;
  }
  return s;
}

// W8A8 gate/up input of the one token, quantized once per workgroup: bf16 values of the codes
// and the block scales.  (Quantizing in each wave at its first expert, with that unit's weight
// loads in flight, needed more registers than a wave has at two waves per SIMD.)
constexpr int kMaxHidden = 8192;
struct ActLds {
  uint32_t xq[kMaxHidden / 2];
  float xs[kMaxHidden / 128];
};

// Thread t takes the 8-value pieces t + NT*j of x [H]; a 128-value block is 16 pieces held by
// 16 consecutive lanes.  Two steps, so that a caller can issue its own loads in between: the
// loads of the pieces, then their quantization into L (the piece count per thread is uniform;
// H is a multiple of 128, so a block never straddles the end).
// J: pieces per thread, at least H / (8 NT).
template <int NT, int J>
struct ActX {
  static constexpr int kJ = J;
  uint4 v[J];
};

template <int NT, int J>
__device__ __forceinline__ void act_x_load(const uint16_t* x, int H, ActX<NT, J>& X) {
  const int n8 = H / 8;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = threadIdx.x + NT * j;
    X.v[j] = c < n8 ? reinterpret_cast<const uint4*>(x)[c] : make_uint4(0, 0, 0, 0);
  }
}

template <int NT, int J>
__device__ __forceinline__ void act_x_quant_store(const ActX<NT, J>& X, int H, ActLds& L) {
  const int n8 = H / 8;
  const int nj = (n8 + NT - 1) / NT;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < nj) {  // uniform: every lane of a wave takes part in the group maximum
      const int c = threadIdx.x + NT * j;
      uint32_t w[4] = {X.v[j].x, X.v[j].y, X.v[j].z, X.v[j].w};
      const float s = act_quant_bf16<16>(w);
      if (c < n8) {
        reinterpret_cast<uint4*>(L.xq)[c] = make_uint4(w[0], w[1], w[2], w[3]);
        if ((c & 15) == 0) L.xs[c >> 4] = s;
      }
    }
  }
}

}  // namespace
}  // namespace moe
