// Router: fp64 logits, top-k by (logit desc, index asc), sigmoid weights renormalized over
// the k routed experts, shared expert fused as the last slot with weight 1.
// blogs.novita.ai, "Optimizing GLM4-MoE for production", section 1 (shared experts fusion:
// top 9 of 161, the shared expert always ninth); molayo1419.me Xiaomi 1T page, section 1
// (sparse top-k routing and its imbalance).  Products of a bf16 and an fp32 value are exact in
// fp64, so ranking on fp64 sums only differs from the reference in summation order.
//
// The sigmoid weights are renormalized over the k routed experts in fp64 and rounded once to
// fp32; the shared expert's weight is exactly 1.
//
// Two launches.  The kernel boundary is the device-wide barrier between the logits and the
// selection: cheaper here than a last-arriving-workgroup handoff, whose arrivals serialize on
// one counter and whose release/acquire fences write back and invalidate the L2.
#include "launch.h"
#include "moe_device.h"
#include "route_select.h"

namespace moe {
namespace {

constexpr int kLogitThreads = 256;
constexpr int kLogitWaves = kLogitThreads / kWave;  // waves split the hidden axis
constexpr int kMaxChunksPerLane = 8;                // hidden <= 8 * 256 * 4

// Logits: workgroup e computes l[t][e] for every token.  Wave w takes the float4 chunks
// c = 64w + lane + 256j of row e of Wr; per lane an fp64 FMA chain over its chunks, then a
// fixed-order DPP reduction per wave, then the waves in order, then the bias.  Tokens go in
// groups of TG with all of a group's activation loads in flight together.
template <int NCH, int TG>
__global__ __launch_bounds__(kLogitThreads) void logits_kernel(RouteArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int H = a.H, M = a.M, E = a.E, e = blockIdx.x;
  const int nc = H / 4;
  __shared__ double part[kLogitWaves][kMaxTokens];
  // Chunk indices are clamped into the row and the surplus masked after the load: every load
  // is unconditional, so all of them are in flight together.
  int cc[NCH];
  bool cv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = wave * kWave + lane + kLogitThreads * j;
    cv[j] = c < nc;
    cc[j] = cv[j] ? c : nc - 1;
  }
  const float4* wr = reinterpret_cast<const float4*>(a.wr + (int64_t)e * H);
  float4 w4[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) w4[j] = wr[cc[j]];
  uint2 xb[TG][NCH];
  auto load_group = [&](int t0) {
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      const int tc = (t0 + tt < M) ? t0 + tt : M - 1;
      const uint2* xt = reinterpret_cast<const uint2*>(a.x + (int64_t)tc * H);
#pragma unroll
      for (int j = 0; j < NCH; ++j) xb[tt][j] = xt[cc[j]];
    }
  };
  load_group(0);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    opaque(w4[j]);
    w4[j] = cv[j] ? w4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int t0 = 0; t0 < M; t0 += TG) {
    if (t0 > 0) load_group(t0);
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        opaque(xb[tt][j]);
        xb[tt][j] = cv[j] ? xb[tt][j] : make_uint2(0, 0);
      }
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].x & 0xFFFF)), (double)w4[j].x, s);
        s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].x >> 16)), (double)w4[j].y, s);
        s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].y & 0xFFFF)), (double)w4[j].z, s);
        s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].y >> 16)), (double)w4[j].w, s);
      }
      s = wave_sum_to_last(s);
      if (lane == kWave - 1 && t0 + tt < M) part[wave][t0 + tt] = s;
    }
  }
  __syncthreads();
  if (wave == 0 && lane < M) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kLogitWaves; ++w) s += part[w][lane];
    if (a.bias) s += (double)a.bias[e];
    a.logits[(int64_t)lane * E + e] = s;
  }
}

// Top-k: workgroup t (one wave) selects token t's experts (wave_select).  One wave per
// workgroup, so the tokens' selections run on different SIMDs rather than sharing one CU's.
template <int KPER>
__global__ __launch_bounds__(kWave) void topk_kernel(RouteArgs a) {
  const int t = blockIdx.x, lane = threadIdx.x % kWave;
  const int E = a.E, S = a.k + a.has_shared;
  if (t >= a.M) return;
  int id;
  float w;
  wave_select<KPER>(a.logits + (int64_t)t * E, E, a.k, a.has_shared, id, w);
  if (lane < S) {
    a.ids[t * S + lane] = id;
    a.w[t * S + lane] = w;
  }
}

template <int NCH>
hipError_t launch_logits(const RouteArgs& a, hipStream_t stream) {
  const dim3 grid(a.E), block(kLogitThreads);
  if (a.M == 1)
    hipLaunchKernelGGL((logits_kernel<NCH, 1>), grid, block, 0, stream, a);
  else if (a.M == 2)
    hipLaunchKernelGGL((logits_kernel<NCH, 2>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((logits_kernel<NCH, 4>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// RMSNorm in front of a layer: one workgroup per token; thread i takes elements i + 1024k.
// Sum of squares in fp64 (exact products; per thread in k order, DPP per wave, waves in order),
// r = 1/sqrt(sum/H + eps), xn = bf16((h * r) * gamma) from fp64 with one rounding.
constexpr int kNormThreads = 1024;
constexpr int kNormPer = 8;  // hidden <= 8192

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(RouteArgs a) {
  __shared__ double part[kNormThreads / kWave];
  const int t = blockIdx.x, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int H = a.H;
  const uint16_t* x = a.x + (int64_t)t * H;
  uint16_t hv[kNormPer];
  float g[kNormPer];
#pragma unroll
  for (int k = 0; k < kNormPer; ++k) {
    const int h = tid + kNormThreads * k;
    const int hc = h < H ? h : H - 1;
    hv[k] = x[hc];
    g[k] = a.gamma[hc];
  }
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < kNormPer; ++k) {
    const double f = bf16_to_f64(hv[k]);
    ss = tid + kNormThreads * k < H ? __fma_rn(f, f, ss) : ss;
  }
  ss = wave_sum_to_last(ss);
  if (lane == kWave - 1) part[wave] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) tot += part[w];
  const double r = 1.0 / sqrt(tot / (double)H + a.eps);
#pragma unroll
  for (int k = 0; k < kNormPer; ++k) {
    const int h = tid + kNormThreads * k;
    if (h < H) {
      a.xn_out[(int64_t)t * H + h] = f64_to_bf16((bf16_to_f64(hv[k]) * r) * (double)g[k]);
      if (a.x_copy) a.x_copy[(int64_t)t * H + h] = hv[k];
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(const RouteArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(a.M), dim3(kNormThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_logits_only(const RouteArgs& a, hipStream_t stream) {
  const int nch = (a.H / 4 + kLogitThreads - 1) / kLogitThreads;
  switch (nch) {
    case 1: return launch_logits<1>(a, stream);
    case 2: return launch_logits<2>(a, stream);
    case 3: return launch_logits<3>(a, stream);
    case 4: return launch_logits<4>(a, stream);
    case 5: return launch_logits<5>(a, stream);
    case 6: return launch_logits<6>(a, stream);
    case 7: return launch_logits<7>(a, stream);
    case 8: return launch_logits<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int nch = (a.H / 4 + kLogitThreads - 1) / kLogitThreads;
  hipError_t err;
  switch (nch) {
    case 1: err = launch_logits<1>(a, stream); break;
    case 2: err = launch_logits<2>(a, stream); break;
    case 3: err = launch_logits<3>(a, stream); break;
    case 4: err = launch_logits<4>(a, stream); break;
    case 5: err = launch_logits<5>(a, stream); break;
    case 6: err = launch_logits<6>(a, stream); break;
    case 7: err = launch_logits<7>(a, stream); break;
    case 8: err = launch_logits<8>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  const int per = (a.E + kWave - 1) / kWave;  // logits per lane in the top-k
  const dim3 grid(a.M), block(kWave);
  if (per <= 3)
    hipLaunchKernelGGL(topk_kernel<3>, grid, block, 0, stream, a);
  else if (per <= 6)
    hipLaunchKernelGGL(topk_kernel<6>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(topk_kernel<(kMaxExperts + kWave - 1) / kWave>, grid, block, 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace moe
