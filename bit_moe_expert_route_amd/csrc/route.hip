// Router: fp64 logits, top-k by (logit desc, index asc), sigmoid weights renormalized over
// the k routed experts, shared expert fused as the last slot with weight 1.
// blogs.novita.ai, "Optimizing GLM4-MoE for production", section 1 (shared experts fusion:
// top 9 of 161, the shared expert always ninth); molayo1419.me Xiaomi 1T page, section 1
// (sparse top-k routing and its imbalance).  Products of a bf16 and an fp32 value are exact in
// fp64, so ranking on fp64 sums only differs from the reference in summation order.
//
// The sigmoid weights are renormalized over the k routed experts in fp64 and rounded once to
// fp32; the shared expert's weight is exactly 1.
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;       // 16
constexpr int kExpertsPerWg = 4;                          // 4 waves per expert
constexpr int kWavesPerExpert = kRouteWaves / kExpertsPerWg;
constexpr int kMaxChunksPerLane = 8;                      // hidden <= 8 * 256 * 4

// One launch.  Workgroup g computes the logits of experts 4g..4g+3 for all M tokens: wave w
// takes expert 4g + w/4 and a quarter of the hidden axis (float4 chunks c = (w%4)*64 + lane +
// 256*j), fp64 accumulation, fixed-order reduction.  The last workgroup to finish (one counter
// in the workspace, a few dozen arrivals) then selects every token's top-k, one wave per token,
// and clears the counter for the next call.
template <int KPER>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int H = a.H, M = a.M, E = a.E;
  const int slot = wave / kWavesPerExpert, quarter = wave % kWavesPerExpert;
  const int e = blockIdx.x * kExpertsPerWg + slot;
  const int nc = H / 4;
  __shared__ double part[kExpertsPerWg][kWavesPerExpert][kMaxTokens];
  __shared__ int last;
  if (e < E) {
    const float4* wr = reinterpret_cast<const float4*>(a.wr + (int64_t)e * H);
    float4 w4[kMaxChunksPerLane];
#pragma unroll
    for (int j = 0; j < kMaxChunksPerLane; ++j) {
      const int c = quarter * kWave + lane + kRouteThreads / kExpertsPerWg * j;
      w4[j] = (c < nc) ? wr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // tokens in pairs: all activation loads of a pair are in flight together
    for (int t0 = 0; t0 < M; t0 += 2) {
      uint2 xb[2][kMaxChunksPerLane];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint2* xt = reinterpret_cast<const uint2*>(a.x + (int64_t)(t0 + tt) * H);
#pragma unroll
        for (int j = 0; j < kMaxChunksPerLane; ++j) {
          const int c = quarter * kWave + lane + kRouteThreads / kExpertsPerWg * j;
          xb[tt][j] = (t0 + tt < M && c < nc) ? xt[c] : make_uint2(0, 0);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if (t0 + tt < M) {
          double s = 0.0;
#pragma unroll
          for (int j = 0; j < kMaxChunksPerLane; ++j) {
            s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].x & 0xFFFF)), (double)w4[j].x, s);
            s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].x >> 16)), (double)w4[j].y, s);
            s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].y & 0xFFFF)), (double)w4[j].z, s);
            s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[tt][j].y >> 16)), (double)w4[j].w, s);
          }
          s = wave_sum(s);
          if (lane == 0) part[slot][quarter][t0 + tt] = s;
        }
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lanes (slot, t): logit of expert 4g+slot for token t, quarters summed in order
    for (int idx = lane; idx < kExpertsPerWg * M; idx += kWave) {
      const int sl = idx / M, t = idx % M, ee = blockIdx.x * kExpertsPerWg + sl;
      if (ee < E) {
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < kWavesPerExpert; ++q) s += part[sl][q][t];
        if (a.bias) s += (double)a.bias[ee];
        a.logits[(int64_t)t * E + ee] = s;
      }
    }
    // publish this workgroup's logits, then count it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(a.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, kWave);
    if (lane == 0) last = (old == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- top-k: wave t selects token t's k best by (logit desc, index asc) ----------------------
  // Each round: lane-local best key, wave maximum (DPP), lowest index holding it.
  const int t = wave;
  if (t < M) {
    const int k = a.k, S = a.k + a.has_shared;
    const double* lt = a.logits + (int64_t)t * E;
    uint64_t key[KPER];
#pragma unroll
    for (int r = 0; r < KPER; ++r) {
      const int ee = lane + kWave * r;
      key[r] = (ee < E) ? f64_key(lt[ee]) : 0ull;  // 0: below every real key
    }
    double my_l = 0.0;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int r = 0; r < KPER; ++r) best = key[r] > best ? key[r] : best;
      const uint64_t kmax = wave_max_u64(best);
      // lowest expert index with the maximum key: lowest r first, then lowest lane
      int r_hit = KPER;
#pragma unroll
      for (int r = KPER - 1; r >= 0; --r)
        if (key[r] == kmax) r_hit = r;
      int r_min = r_hit;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const int other = __shfl_xor(r_min, o, kWave);
        r_min = other < r_min ? other : r_min;
      }
      const uint64_t lanes = __ballot(r_hit == r_min);
      const int win_lane = __builtin_ctzll(lanes);
      const int idx = win_lane + kWave * r_min;
#pragma unroll
      for (int r = 0; r < KPER; ++r)
        if (lane == win_lane && r == r_min) key[r] = 0;
      if (lane == j) { my_i = idx; my_l = lt[idx]; }
    }
    // weights: sigmoid per slot in its lane, sum in slot order
    const double sg = (lane < k) ? 1.0 / (1.0 + exp(-my_l)) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += __shfl(sg, j, kWave);
    if (lane < k) {
      a.ids[t * S + lane] = my_i;
      a.w[t * S + lane] = __double2float_rn(sg / sum);
    }
    if (a.has_shared && lane == 0) {
      a.ids[t * S + k] = E;
      a.w[t * S + k] = 1.0f;
    }
  }
  if (tid == 0) __hip_atomic_store(a.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int grid = (a.E + kExpertsPerWg - 1) / kExpertsPerWg;
  const int per = (a.E + kWave - 1) / kWave;  // logits per lane in the top-k
  if (per <= 4)
    hipLaunchKernelGGL(route_kernel<4>, dim3(grid), dim3(kRouteThreads), 0, stream, a);
  else if (per <= 8)
    hipLaunchKernelGGL(route_kernel<8>, dim3(grid), dim3(kRouteThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(route_kernel<(kMaxExperts + kWave - 1) / kWave>, dim3(grid),
                       dim3(kRouteThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
