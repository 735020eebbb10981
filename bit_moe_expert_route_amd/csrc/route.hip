// Router: fp64 logits, top-k by (logit desc, index asc), sigmoid weights renormalized over
// the k routed experts, shared expert fused as the last slot with weight 1.
// blogs.novita.ai, "Optimizing GLM4-MoE for production", section 1 (shared experts fusion:
// top 9 of 161, the shared expert always ninth); molayo1419.me Xiaomi 1T page, section 1
// (sparse top-k routing and its imbalance).  Products of a bf16 and an fp32 value are exact in
// fp64, so ranking on fp64 sums only differs from the reference in summation order.
//
// Two launches: workgroup e computes logit e for all M tokens; then one wave per token selects
// its top-k.  (A last-arriver counter would save the second launch but costs more in
// device-scope atomics and fences than the launch.)
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;

// Logits of one routed expert e for all M tokens: l[t][e] = sum_h x[t][h] * Wr[e][h] (+ b[e]).
// Thread tid covers float4 chunks c = tid + 256*j (all issued before use); fixed-order wave
// and cross-wave reduction.
constexpr int kMaxChunksPerThread = 8;  // hidden <= 8 * 256 * 4
__global__ __launch_bounds__(kRouteThreads) void route_logits_kernel(RouteArgs a) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int H = a.H, M = a.M, E = a.E;
  const int nc = H / 4;
  const float4* wr = reinterpret_cast<const float4*>(a.wr + (int64_t)e * H);
  float4 w4[kMaxChunksPerThread];
#pragma unroll
  for (int j = 0; j < kMaxChunksPerThread; ++j) {
    const int c = tid + kRouteThreads * j;
    w4[j] = (c < nc) ? wr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __shared__ double part[kRouteWaves][kMaxTokens];
  for (int t = 0; t < M; ++t) {
    const uint2* xt = reinterpret_cast<const uint2*>(a.x + (int64_t)t * H);
    uint2 xb[kMaxChunksPerThread];
#pragma unroll
    for (int j = 0; j < kMaxChunksPerThread; ++j) {
      const int c = tid + kRouteThreads * j;
      xb[j] = (c < nc) ? xt[c] : make_uint2(0, 0);
    }
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxChunksPerThread; ++j) {
      s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].x & 0xFFFF)), (double)w4[j].x, s);
      s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].x >> 16)), (double)w4[j].y, s);
      s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].y & 0xFFFF)), (double)w4[j].z, s);
      s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].y >> 16)), (double)w4[j].w, s);
    }
    s = wave_sum(s);
    if (lane == 0) part[wave][t] = s;
  }
  __syncthreads();
  if (tid < M) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) s += part[w][tid];
    if (a.bias) s += (double)a.bias[e];
    a.logits[(int64_t)tid * E + e] = s;
  }
}

// Top-k of token t: k rounds of a wave arg-max over (logit desc, index asc) on the logits held
// in registers (up to 17 per lane); lane j keeps slot j; weights sigmoid(l)/sum in fp64.
__global__ __launch_bounds__(kWave) void route_topk_kernel(RouteArgs a) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int E = a.E, k = a.k, S = a.k + a.has_shared;
  constexpr int kPer = (kMaxExperts + kWave - 1) / kWave;
  const double* lt = a.logits + (int64_t)t * E;
  double v[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int ee = lane + kWave * r;
    v[r] = (ee < E) ? lt[ee] : 0.0;
  }
  uint32_t taken = 0;  // bit r: candidate r of this lane already selected
  double sig_sum = 0.0, my_l = 0.0;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    double bv = 0.0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int ee = lane + kWave * r;
      const bool cand = ee < E && !((taken >> r) & 1u);
      if (cand && (bi == 0x7FFFFFFF || v[r] > bv)) { bv = v[r]; bi = ee; }  // ascending ee
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      const bool take = (oi != 0x7FFFFFFF) &&
                        (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi));
      if (take) { bv = ov; bi = oi; }
    }
    if ((bi % kWave) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) { my_l = bv; my_i = bi; }
    sig_sum += 1.0 / (1.0 + exp(-bv));
  }
  if (lane < k) {
    a.ids[t * S + lane] = my_i;
    a.w[t * S + lane] = __double2float_rn((1.0 / (1.0 + exp(-my_l))) / sig_sum);
  }
  if (a.has_shared && lane == 0) {
    a.ids[t * S + k] = E;
    a.w[t * S + k] = 1.0f;
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(route_logits_kernel, dim3(a.E), dim3(kRouteThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_topk_kernel, dim3(a.M), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
