// Fused QK-norm + RoPE: the attention-side pre-norms of a decode step in one kernel.
//   blogs.novita.ai "Optimizing GLM4-MoE for production", section 2 (QKNorm fusion): the
//   head-wise RMSNorm of Q and K and the rotary embedding are both per-head computations, so
//   one kernel does both; in the GLM4-MoE variant only half of each head's dimensions rotate.
//   molayo1419.me Xiaomi 1T page, section 1: RMSNorm and RoPE are among the per-layer operators
//   whose boundaries (launch, barrier, HBM round trip) dominate at high token rates.
// Per token t and head h (query heads [0, nq) with gamma_q, key heads [nq, nq + nk) with
// gamma_k), over the head's hd values x (the half-split pairing is a reading, the pages name
// none):
//   r = 1/sqrt(sum(x^2)/hd + eps);  n_k = (x_k * r) * gamma_k;
//   for i < rot/2, angle = pos_t * theta^(-2i/rot), c = cos, s = sin:
//     y_i = n_i c - n_{i+rot/2} s,   y_{i+rot/2} = n_{i+rot/2} c + n_i s;   y_k = n_k for k >= rot.
// All in fp64 (exact bf16 inputs and fp32 gains), each output rounded once to bf16, in place.
//
// Layout: one workgroup per (token, 4 heads), one wave per head, lane l holding the E = hd/64
// consecutive values [E l, E l + E) (one 2-, 4- or 8-byte load).  The rot/2 angles of the token
// are computed once per workgroup (fp64 sincos) into LDS; a value's rotation partner sits rot/2
// values away, so E rot/2-aligned values of a lane pair with the same lane.  Bound: latency (a
// 16-token GLM-shaped call moves 425 KB).
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kQkThreads = 256;
constexpr int kQkHeadsPerBlock = kQkThreads / kWave;
constexpr int kQkMaxHalf = 128;  // rot/2 <= hd/2 <= 128

template <int E>
struct Packed;
template <>
struct Packed<1> { using T = uint16_t; };
template <>
struct Packed<2> { using T = uint32_t; };
template <>
struct Packed<4> { using T = uint2; };

template <int E>
__device__ __forceinline__ void unpack(const typename Packed<E>::T& p, uint16_t (&v)[E]) {
  if constexpr (E == 1) {
    v[0] = p;
  } else if constexpr (E == 2) {
    v[0] = (uint16_t)p;
    v[1] = (uint16_t)(p >> 16);
  } else {
    v[0] = (uint16_t)p.x;
    v[1] = (uint16_t)(p.x >> 16);
    v[2] = (uint16_t)p.y;
    v[3] = (uint16_t)(p.y >> 16);
  }
}

template <int E>
__device__ __forceinline__ typename Packed<E>::T pack(const uint16_t (&v)[E]) {
  if constexpr (E == 1) return v[0];
  else if constexpr (E == 2) return (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  else return make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                         (uint32_t)v[2] | ((uint32_t)v[3] << 16));
}

// Sum over the wave, every lane gets it (butterfly order, fixed).
__device__ __forceinline__ double wave_allsum(double v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <int E>
__global__ __launch_bounds__(kQkThreads) void qk_norm_rope_kernel(QkRopeArgs a) {
  __shared__ double cs_c[kQkMaxHalf], cs_s[kQkMaxHalf];
  const int t = blockIdx.x;
  const int half = a.rot / 2;
  if ((int)threadIdx.x < half) {
    const double ang = (double)a.pos[t] * pow(a.theta, -2.0 * (double)threadIdx.x / (double)a.rot);
    double sn, c;
    sincos(ang, &sn, &c);
    cs_c[threadIdx.x] = c;
    cs_s[threadIdx.x] = sn;
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int h = blockIdx.y * kQkHeadsPerBlock + wave;
  const bool live = h < a.nq + a.nk;
  using P = typename Packed<E>::T;
  P* ptr = reinterpret_cast<P*>(a.qk + (int64_t)t * a.stride + (int64_t)(live ? h : 0) * a.hd) +
           lane;
  uint16_t xv[E];
  unpack<E>(*ptr, xv);
  const float* g = h < a.nq ? a.gamma_q : a.gamma_k;
  double n[E];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const double v = bf16_to_f64(xv[k]);
    ss += v * v;
  }
  ss = wave_allsum(ss);
  const double r = 1.0 / sqrt(ss / (double)a.hd + a.eps);
#pragma unroll
  for (int k = 0; k < E; ++k) n[k] = (bf16_to_f64(xv[k]) * r) * (double)g[E * lane + k];
  __syncthreads();  // the angles
  // the rotation partner of value e = E lane + k is e +- half, in lane lane +- half / E
  const int e0 = E * lane;
  const bool rotated = e0 < a.rot;
  const bool low = e0 < half;
  const int partner = rotated ? (low ? lane + half / E : lane - half / E) : lane;
  uint16_t yv[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const double np = __shfl(n[k], partner, kWave);
    double y = n[k];
    if (rotated) {
      const int i = (low ? e0 : e0 - half) + k;
      y = low ? n[k] * cs_c[i] - np * cs_s[i] : n[k] * cs_c[i] + np * cs_s[i];
    }
    yv[k] = f64_to_bf16(y);
  }
  if (live) *ptr = pack<E>(yv);
}

}  // namespace

hipError_t launch_qk_norm_rope(const QkRopeArgs& a, hipStream_t stream) {
  const int nh = a.nq + a.nk;
  const dim3 grid((unsigned)a.M, (unsigned)((nh + kQkHeadsPerBlock - 1) / kQkHeadsPerBlock));
  switch (a.hd) {
    case 64:
      hipLaunchKernelGGL(qk_norm_rope_kernel<1>, grid, dim3(kQkThreads), 0, stream, a);
      break;
    case 128:
      hipLaunchKernelGGL(qk_norm_rope_kernel<2>, grid, dim3(kQkThreads), 0, stream, a);
      break;
    case 256:
      hipLaunchKernelGGL(qk_norm_rope_kernel<4>, grid, dim3(kQkThreads), 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
