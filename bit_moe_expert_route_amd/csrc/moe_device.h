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

// FP8_B128_A8: FP8_B128 weights with the activations quantized live (W8A8)
enum { WFMT_MXFP4 = 1, WFMT_FP8_B128 = 2, WFMT_FP8_B128_A8 = 3 };

// ---- element formats -------------------------------------------------------------------

// E8M0 block exponent -> fp32 2^(s-127); 0 -> 2^-127 (subnormal); 255 -> NaN.  Branch-free
// (selects), so it can sit in a load/compute pipeline without splitting it.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7FC00000u : bits;
  return __uint_as_float(bits);
}

// Magnitude t >= 0 (fp32) -> E4M3FN magnitude code, nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
  if (t >= 448.0f) return 0x7E;
  if (t < 0x1p-6f) {
    // subnormal range: spacing 2^-9; t*512 is exact, rintf rounds ties to even
    return (uint32_t)rintf(t * 512.0f);  // 8 -> code 8 = 2^-6, the first normal
  }
  const uint32_t u = __float_as_uint(t);
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;  // exponent:3-bit mantissa, RNE
  uint32_t code = r - ((127u - 7u) << 3);
  return code > 0x7Eu ? 0x7Eu : code;
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
// with every decoded value kept live (which would cost far more registers than it saves), and
// right after a load whose value is masked later, so that the load is not sunk into a branch
// (a load inside a branch is waited for inside it, which serializes the loads).
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ void opaque(float4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void opaque(uint2& v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }
__device__ __forceinline__ void opaque(double& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(int& v) { asm volatile("" : "+v"(v)); }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8-byte streaming load (non-temporal hint).
__device__ __forceinline__ uint2 load_stream8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
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

// fp64 -> bf16 bits, one rounding to nearest even of the double's exact value (no double
// rounding): round to odd at fp32 precision (the nearest-even fp32 stepped toward zero when it
// rounded away, with its last bit set when inexact), then nearest-even to bf16; 24 bits are
// at least two more than bf16's 8, which makes the two steps equal to one direct rounding.
// Overflow gives infinity and NaN stays NaN.
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
  float f = (float)d;
  const double back = (double)f;
  if (back != d && d == d) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(d)) u -= 1u;
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f32_to_bf16(f);
}

__device__ __forceinline__ double bf16_to_f64(uint16_t b) { return (double)bf16_to_f32(b); }

// ---- wavefront reductions ----------------------------------------------------------------

// DPP move of v (as bits) with control CTRL on rows ROWMASK; lanes without a source read 0.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xf,
                                                    false));
}

// Sum over the 64 lanes, fixed order, result valid in lane 63 only: shifts within each 16-lane
// row (row_shr 1, 2, 4, 8), then row 15 -> rows 1, 3 and lane 31 -> rows 2, 3 broadcasts.
// VALU data-parallel moves, no LDS round trips.
__device__ __forceinline__ float wave_sum_to_last(float v) {
  v += dpp0<0x111>(v);
  v += dpp0<0x112>(v);
  v += dpp0<0x114>(v);
  v += dpp0<0x118>(v);
  v += dpp0<0x142, 0xa>(v);
  v += dpp0<0x143, 0xc>(v);
  return v;
}

// Monotone map of a double to an unsigned key (larger value -> larger key; -0 < +0).
__device__ __forceinline__ uint64_t f64_key(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWMASK, 0xf, false);
}

// Wave-wide maximum / minimum of a 32-bit unsigned value, returned wave-uniform (lanes without
// a DPP source read 0, the identity of the maximum; the minimum works on the complement).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111>(v, 0));
  v = max(v, dpp_u32<0x112>(v, 0));
  v = max(v, dpp_u32<0x114>(v, 0));
  v = max(v, dpp_u32<0x118>(v, 0));
  v = max(v, dpp_u32<0x142, 0xa>(v, 0));
  v = max(v, dpp_u32<0x143, 0xc>(v, 0));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// fp64 version of wave_sum_to_last: same fixed order, result valid in lane 63 only.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ double dpp0(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t hi = dpp_u32<CTRL, ROWMASK>((uint32_t)(b >> 32), 0);
  const uint32_t lo = dpp_u32<CTRL, ROWMASK>((uint32_t)b, 0);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum_to_last(double v) {
  v += dpp0<0x111>(v);
  v += dpp0<0x112>(v);
  v += dpp0<0x114>(v);
  v += dpp0<0x118>(v);
  v += dpp0<0x142, 0xa>(v);
  v += dpp0<0x143, 0xc>(v);
  return v;
}

// Inverse of f64_key.
__device__ __forceinline__ double f64_from_key(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}

// Lane l's value of a wave-varying double, returned wave-uniform.
__device__ __forceinline__ double read_lane(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---- expert-sorted work queue, one copy per wave ------------------------------------------
// Each wave derives, from the M*S routing ids, the ascending list of distinct active experts
// ("ranks") and, for each, the (token, slot) pairs that selected it, without any workgroup
// barrier: pair i lives in lane i % 64, register i / 64; an LDS bitmap (per wave) gives every
// expert its rank by a prefix count.  Ids outside [0, n_experts) are ignored and flagged.
constexpr int kPairRegs = kMaxPairs / kWave;

struct WaveQueue {
  int e[kPairRegs];     // this lane's pairs: expert id, or -1
  int rank[kPairRegs];  // rank of that expert among the active ones, or -1
  int n_active;         // wave-uniform
  bool invalid;         // wave-uniform: some id was out of range
  uint32_t* bits;       // LDS bitmap of active experts [kBitmapWords]
  int* base;            // LDS: active experts before each bitmap word [kBitmapWords]
};

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// The queue from the ids of pairs lane + 64k held in v[k] (pairs >= n_pairs ignored).
__device__ __forceinline__ void wave_queue_from(WaveQueue& Q, uint32_t* bits, int* base,
                                                int (&v)[kPairRegs], int n_pairs,
                                                int n_experts) {
  const int lane = threadIdx.x % kWave;
  Q.bits = bits;
  Q.base = base;
  if (lane < kBitmapWords) bits[lane] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  int inv = 0;
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k) {
    opaque(v[k]);
    const bool in = lane + kWave * k < n_pairs;
    const bool ok = v[k] >= 0 && v[k] < n_experts;
    Q.e[k] = (in && ok) ? v[k] : -1;
    inv |= (in && !ok) ? 1 : 0;
  }
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k)
    if (Q.e[k] >= 0) atomicOr(&bits[Q.e[k] >> 5], 1u << (Q.e[k] & 31));
  Q.invalid = __ballot(inv) != 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int pc = (lane < kBitmapWords) ? __popc(bits[lane]) : 0;
  const int incl = wave_inclusive_scan(pc, lane);
  if (lane < kBitmapWords) base[lane] = incl - pc;
  Q.n_active = __shfl(incl, kWave - 1, kWave);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k) {
    const int e = Q.e[k], w = (e >= 0 ? e : 0) >> 5;
    const int r = base[w] + __popc(bits[w] & ((1u << (e & 31)) - 1u));
    Q.rank[k] = (e >= 0) ? r : -1;
  }
}

// The queue from the routing ids in global memory [n_pairs].
__device__ __forceinline__ void wave_queue_build(WaveQueue& Q, uint32_t* bits, int* base,
                                                 const int32_t* __restrict__ ids, int n_pairs,
                                                 int n_experts) {
  const int lane = threadIdx.x % kWave;
  // all id loads in flight together (clamped index, masked after the load)
  int v[kPairRegs];
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k) {
    const int i = lane + kWave * k;
    v[k] = ids[i < n_pairs ? i : n_pairs - 1];
  }
  wave_queue_from(Q, bits, base, v, n_pairs, n_experts);
}

// Cost-weighted split of the expert-major unit list (expert rank q owns units
// [q*upe, (q+1)*upe)) over the waves of a grid.  A unit of an expert selected by m pairs costs
// base + extra*(m-1): every extra pair adds a pass over the unit's weights with another token's
// activations.  Wave g takes the units whose start position in the cost order lies in
// [C*g/NW, C*(g+1)/NW), so a wave holding units of the shared expert (M pairs) holds
// proportionally fewer of them.  Lane l describes experts q = 4l..4l+3.
struct WaveBalance {
  int pre[4];   // exclusive prefix cost of expert 4l+j
  int cost[4];  // cost of one unit of expert 4l+j
  int total;    // wave-uniform total cost
  int upe;      // units per expert
  int n_active;
};

__device__ __forceinline__ void wave_balance_build(WaveBalance& B, const WaveQueue& Q, int* cnt,
                                                   int upe, int base, int extra) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < 4; ++j) cnt[4 * lane + j] = 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k)
    if (Q.rank[k] >= 0) atomicAdd(&cnt[Q.rank[k]], 1);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 4 * lane + j;
    const int m = cnt[q];
    B.cost[j] = q < Q.n_active ? base + extra * (m - 1) : 0;
    sum += B.cost[j] * upe;
  }
  const int incl = wave_inclusive_scan(sum, lane);
  int run = incl - sum;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    B.pre[j] = run;
    run += B.cost[j] * upe;
  }
  B.total = __shfl(incl, kWave - 1, kWave);
  B.upe = upe;
  B.n_active = Q.n_active;
}

// First unit whose start position in the cost order is >= pos (pos wave-uniform).
__device__ __forceinline__ int wave_balance_unit(const WaveBalance& B, int64_t pos) {
  if (pos >= B.total) return B.n_active * B.upe;
  const int lane = threadIdx.x % kWave;
  const uint64_t has = __ballot(4 * lane < B.n_active && B.pre[0] <= pos);
  const int L = 63 - __builtin_clzll(has);  // pos >= pre of expert 0 = 0, so has != 0
  int jsel = 0;
#pragma unroll
  for (int j = 1; j < 4; ++j)
    if (4 * lane + j < B.n_active && B.pre[j] <= pos) jsel = j;
  int mp = B.pre[0], mc = B.cost[0];
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    mp = jsel == j ? B.pre[j] : mp;
    mc = jsel == j ? B.cost[j] : mc;
  }
  const int q = 4 * L + __builtin_amdgcn_readlane(jsel, L);
  const int P = __builtin_amdgcn_readlane(mp, L);
  const int c = __builtin_amdgcn_readlane(mc, L);
  const int i = (int)(((int64_t)pos - P + c - 1) / c);
  return q * B.upe + i;  // i == upe is the next expert's first unit
}

// Expert id of rank q (q < n_active).  Wave-uniform.
__device__ __forceinline__ int wave_queue_expert(const WaveQueue& Q, int q) {
  const int lane = threadIdx.x % kWave;
  bool hit = false;
  if (lane < kBitmapWords) {
    const int b = Q.base[lane];
    hit = b <= q && q < b + __popc(Q.bits[lane]);
  }
  const uint64_t m = __ballot(hit);
  const int w = __builtin_ctzll(m);
  uint32_t word = Q.bits[w];
  for (int r = q - Q.base[w]; r > 0; --r) word &= word - 1u;
  return (w << 5) + __builtin_ctz(word);
}

// Pairs of rank q as bit masks: bit l of mask k <=> pair l + 64k.
__device__ __forceinline__ void wave_queue_pairs(const WaveQueue& Q, int q,
                                                 uint64_t (&mask)[kPairRegs]) {
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k) mask[k] = __ballot(Q.rank[k] == q);
}

// Lowest pair index in the masks (the masks are non-empty).
__device__ __forceinline__ int first_pair(const uint64_t (&mask)[kPairRegs]) {
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k)
    if (mask[k]) return kWave * k + __builtin_ctzll(mask[k]);
  return 0;
}

}  // namespace moe
