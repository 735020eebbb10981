// Router: fp64 logits, top-k by (logit desc, index asc), sigmoid weights renormalized over
// the k routed experts, shared expert fused as the last slot with weight 1.
// blogs.novita.ai, "Optimizing GLM4-MoE for production", section 1 (shared experts fusion:
// top 9 of 161, the shared expert always ninth); molayo1419.me Xiaomi 1T page, section 1
// (sparse top-k routing and its imbalance).  Products of a bf16 and an fp32 value are exact in
// fp64, so ranking on fp64 sums only differs from the reference in summation order.
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;

// One workgroup per routed expert e: l[t][e] = sum_h x[t][h] * Wr[e][h] (+ b[e]) for all M
// tokens; each thread strides over h, then a fixed-order wave and cross-wave reduction.
__global__ __launch_bounds__(kRouteThreads) void router_logits_kernel(
    const uint16_t* __restrict__ x, int M, int H, const float* __restrict__ wr,
    const float* __restrict__ bias, int E, double* __restrict__ logits) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  double acc[kMaxTokens];
#pragma unroll
  for (int t = 0; t < kMaxTokens; ++t) acc[t] = 0.0;
  const float* row = wr + (int64_t)e * H;
  for (int h = tid; h < H; h += kRouteThreads) {
    const double wv = (double)row[h];
#pragma unroll
    for (int t = 0; t < kMaxTokens; ++t)
      if (t < M) acc[t] = __fma_rn((double)bf16_to_f32(x[(int64_t)t * H + h]), wv, acc[t]);
  }
  __shared__ double part[kRouteThreads / kWave][kMaxTokens];
  const int wave = tid / kWave, lane = tid % kWave;
#pragma unroll
  for (int t = 0; t < kMaxTokens; ++t) {
    if (t < M) {
      const double v = wave_sum(acc[t]);
      if (lane == 0) part[wave][t] = v;
    }
  }
  __syncthreads();
  if (tid < M) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kRouteThreads / kWave; ++w) s += part[w][tid];
    if (bias) s += (double)bias[e];
    logits[(int64_t)tid * E + e] = s;
  }
}

// One workgroup per token: rank of every expert by (logit desc, index asc); the k best fill
// the slots in rank order, then weights sigmoid(l)/sum over the k, in fp64.
__global__ __launch_bounds__(kRouteThreads) void router_topk_kernel(
    const double* __restrict__ logits, int E, int k, int has_shared,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int S = k + has_shared;
  __shared__ double l[kMaxExperts];
  __shared__ int sel[kMaxSlots];
  for (int e = tid; e < E; e += kRouteThreads) l[e] = logits[(int64_t)t * E + e];
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    const double le = l[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const double lf = l[f];
      rank += (lf > le) || (lf == le && f < e);
    }
    if (rank < k) sel[rank] = e;
  }
  __syncthreads();
  if (tid == 0) {
    double sig[kMaxSlots];
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
      sig[j] = 1.0 / (1.0 + exp(-l[sel[j]]));
      sum += sig[j];
    }
    for (int j = 0; j < k; ++j) {
      ids[t * S + j] = sel[j];
      w[t * S + j] = __double2float_rn(sig[j] / sum);
    }
    if (has_shared) {
      ids[t * S + k] = E;
      w[t * S + k] = 1.0f;
    }
  }
}

}  // namespace

hipError_t launch_route(const uint16_t* x, int M, int H, const float* wr, const float* bias,
                        int E, int k, int has_shared, int32_t* ids, float* w, double* logits,
                        hipStream_t stream) {
  hipLaunchKernelGGL(router_logits_kernel, dim3(E), dim3(kRouteThreads), 0, stream, x, M, H,
                     wr, bias, E, logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(router_topk_kernel, dim3(M), dim3(kRouteThreads), 0, stream, logits, E, k,
                     has_shared, ids, w);
  return hipGetLastError();
}

}  // namespace moe
