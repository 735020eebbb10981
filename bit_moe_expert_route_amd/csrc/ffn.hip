// Expert FFN decode: stream each active expert's packed W13 and W2 once, SwiGLU in between,
// weighted combine in slot order.
//   molayo1419.me Xiaomi 1T page, section 1: decode reads every active weight from HBM once per
//   step and is bound by bandwidth; section 2: expert FFN weights in MXFP4.
//   d9249.github.io "glm-5-2-b300-kernel-mtp-serving", table under "what it solves" and idea 1:
//   a batch-1 expert GEMM needs many concurrent memory streams per compute unit to approach
//   peak bandwidth; idea 3: a verify block of M tokens shares one weight stream.
//   blogs.novita.ai "Optimizing GLM4-MoE for production", section 1: the shared expert runs as
//   one more slot of the same fused MoE.
//
// Work decomposition (one launch per phase):
//   gate/up  : item = (active expert q, block of IB intermediate indices); each wave owns two
//              indices i, i' and streams the four rows gate_i, up_i, gate_i', up_i' with lanes
//              across 16-byte chunks of K = H; a = silu(g) * u goes to the workspace.
//   down     : item = (active expert q, block of HB output rows); each wave streams RPW rows of
//              W2 at a time, lanes across 16-byte chunks of K = I; o goes to the workspace.
//   combine  : y[t][h] = sum_j w[t][j] * o[t][j][h] in slot order, rounded to bf16.
// Activations of the expert's tokens are staged in LDS (bf16 x, fp32 a), TG tokens at a time;
// each 16-byte weight chunk is decoded once per token in registers (hardware E2M1/E4M3 -> bf16
// or fp32 conversion), block scales are applied to each chunk's partial sum.
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kFfnThreads = 256;
constexpr int kWaves = kFfnThreads / kWave;

template <int FMT>
struct Fmt;
template <>
struct Fmt<WFMT_FP8_B128> {
  static constexpr int kVals = 16;  // values per 16-byte chunk
  __device__ static int64_t row_bytes(int K) { return K; }
};
template <>
struct Fmt<WFMT_MXFP4> {
  static constexpr int kVals = 32;
  __device__ static int64_t row_bytes(int K) { return K / 2; }
};

// Block scale of chunk c of row r of one expert matrix [R][K].
template <int FMT>
__device__ __forceinline__ float chunk_scale(const void* scales, int R, int K, int r, int c);
template <>
__device__ __forceinline__ float chunk_scale<WFMT_FP8_B128>(const void* scales, int R, int K,
                                                            int r, int c) {
  (void)R;
  return reinterpret_cast<const float*>(scales)[(r >> 7) * (K >> 7) + (c >> 3)];
}
template <>
__device__ __forceinline__ float chunk_scale<WFMT_MXFP4>(const void* scales, int R, int K, int r,
                                                         int c) {
  (void)R;
  return e8m0_to_f32(reinterpret_cast<const uint8_t*>(scales)[(int64_t)r * (K >> 5) + c]);
}

// Scale storage of one expert matrix [R][K], in elements of the scale type.
template <int FMT>
__device__ __forceinline__ int64_t scale_elems(int R, int K) {
  return FMT == WFMT_FP8_B128 ? (int64_t)(R >> 7) * (K >> 7) : (int64_t)R * (K >> 5);
}

template <int FMT>
__device__ __forceinline__ const void* scale_ptr(const void* base, int64_t elems_before) {
  if (FMT == WFMT_FP8_B128) return reinterpret_cast<const float*>(base) + elems_before;
  return reinterpret_cast<const uint8_t*>(base) + elems_before;
}

// Sum over one 16-byte weight chunk times bf16 activations (16 or 32 values) read from LDS.
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16(uint4 wq, const uint16_t* xs) {
  const uint4* xv = reinterpret_cast<const uint4*>(xs);
  float acc = 0.0f;
  if constexpr (FMT == WFMT_FP8_B128) {
    const uint4 x0 = xv[0], x1 = xv[1];
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x2 lo, hi;
      fp8x4_to_bf16(ww[j], lo, hi);
      acc = dot2(lo, as_bf16x2(xw[2 * j]), acc);
      acc = dot2(hi, as_bf16x2(xw[2 * j + 1]), acc);
    }
  } else {
    const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 xq = xv[j];
      const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w};
      bf16x2 wb[4];
      fp4x8_to_bf16(ww[j], wb);
#pragma unroll
      for (int b = 0; b < 4; ++b) acc = dot2(wb[b], as_bf16x2(xw[b]), acc);
    }
  }
  return acc;
}

// Sum over one 16-byte weight chunk times fp32 activations read from LDS.
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32(uint4 wq, const float* as) {
  const float4* av = reinterpret_cast<const float4*>(as);
  const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
  float acc = 0.0f;
  if constexpr (FMT == WFMT_FP8_B128) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a4 = av[j];
      const f32x2 lo = fp8x2_to_f32<false>(ww[j]), hi = fp8x2_to_f32<true>(ww[j]);
      acc = __builtin_fmaf(lo.x, a4.x, acc);
      acc = __builtin_fmaf(lo.y, a4.y, acc);
      acc = __builtin_fmaf(hi.x, a4.z, acc);
      acc = __builtin_fmaf(hi.y, a4.w, acc);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a0 = av[2 * j], a1 = av[2 * j + 1];
      const f32x2 p0 = fp4x2_to_f32<0>(ww[j]), p1 = fp4x2_to_f32<1>(ww[j]);
      const f32x2 p2 = fp4x2_to_f32<2>(ww[j]), p3 = fp4x2_to_f32<3>(ww[j]);
      acc = __builtin_fmaf(p0.x, a0.x, acc);
      acc = __builtin_fmaf(p0.y, a0.y, acc);
      acc = __builtin_fmaf(p1.x, a0.z, acc);
      acc = __builtin_fmaf(p1.y, a0.w, acc);
      acc = __builtin_fmaf(p2.x, a1.x, acc);
      acc = __builtin_fmaf(p2.y, a1.y, acc);
      acc = __builtin_fmaf(p3.x, a1.z, acc);
      acc = __builtin_fmaf(p3.y, a1.w, acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return (g / (1.0f + __expf(-g))) * u;
}

// ---- gate/up + SwiGLU ----------------------------------------------------------------------
template <int FMT, int NS>
__global__ __launch_bounds__(kFfnThreads) void gateup_kernel(FfnArgs a) {
  __shared__ QueueLds Q;
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn_lds);

  const int q = blockIdx.x / a.items13, item = blockIdx.x % a.items13;
  const int e = build_queue(Q, a.ids, a.M * a.S, a.n_experts, q);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  if (e < 0) return;

  const int H = a.H, I = a.I, R = 2 * I;
  constexpr int V = Fmt<FMT>::kVals;
  const int C = H / V;  // 16-byte chunks per row
  const int64_t rb = Fmt<FMT>::row_bytes(H);
  const uint8_t* W = a.w13 + (int64_t)e * R * rb;
  const void* Ws = scale_ptr<FMT>(a.w13s, (int64_t)e * scale_elems<FMT>(R, H));
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int i0 = item * a.ib + wave * 2;  // this wave's two intermediate indices i0, i0+1
  const bool active = i0 < (item + 1) * a.ib;

  // Issue all weight loads of the wave's four rows before touching LDS.
  uint4 wq[4][NS];
  float ws[4][NS];
  if (active) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (r & 1) * I + i0 + (r >> 1);  // gate_i0, up_i0, gate_i0+1, up_i0+1
      const uint4* src = reinterpret_cast<const uint4*>(W + (int64_t)row * rb);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = lane + kWave * s;
        if (c < C) {
          wq[r][s] = load_stream16(src + c);
          ws[r][s] = chunk_scale<FMT>(Ws, R, H, row, c);
        } else {
          wq[r][s] = make_uint4(0, 0, 0, 0);
          ws[r][s] = 0.0f;
        }
      }
    }
  }

  const int m = Q.n_pairs;
  for (int t0 = 0; t0 < m; t0 += a.tg13) {
    const int tn = min(a.tg13, m - t0);
    __syncthreads();  // previous tile fully consumed
    // stage x of tokens t0..t0+tn into LDS
    const int vec_per_tok = H / 8;  // uint4 of 8 bf16
    for (int v = threadIdx.x; v < tn * vec_per_tok; v += kFfnThreads) {
      const int tt = v / vec_per_tok, off = v % vec_per_tok;
      const int tok = Q.pairs[t0 + tt] / a.S;
      reinterpret_cast<uint4*>(xs + (int64_t)tt * H)[off] =
          reinterpret_cast<const uint4*>(a.x + (int64_t)tok * H)[off];
    }
    __syncthreads();
    if (!active) continue;
    for (int tt = 0; tt < tn; ++tt) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* xt = xs + (int64_t)tt * H;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = lane + kWave * s;
        if (c < C) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[r] = __builtin_fmaf(chunk_dot_bf16<FMT>(wq[r][s], xt + c * V), ws[r][s], acc[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = wave_sum(acc[r]);
      if (lane == 0) {
        const int p = Q.pairs[t0 + tt];
        float* dst = a.a_buf + (int64_t)p * I;
        dst[i0] = silu_mul(acc[0], acc[1]);
        dst[i0 + 1] = silu_mul(acc[2], acc[3]);
      }
    }
  }
}

// ---- down projection -----------------------------------------------------------------------
template <int FMT, int NS, int RPW>
__global__ __launch_bounds__(kFfnThreads) void down_kernel(FfnArgs a) {
  __shared__ QueueLds Q;
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  float* as = reinterpret_cast<float*>(dyn_lds);

  const int q = blockIdx.x / a.items2, item = blockIdx.x % a.items2;
  const int e = build_queue(Q, a.ids, a.M * a.S, a.n_experts, q);
  if (e < 0) return;

  const int H = a.H, I = a.I;
  constexpr int V = Fmt<FMT>::kVals;
  const int C = I / V;
  const int64_t rb = Fmt<FMT>::row_bytes(I);
  const uint8_t* W = a.w2 + (int64_t)e * H * rb;
  const void* Ws = scale_ptr<FMT>(a.w2s, (int64_t)e * scale_elems<FMT>(H, I));
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int h_begin = item * a.hb, h_end = h_begin + a.hb;

  const int m = Q.n_pairs;
  for (int t0 = 0; t0 < m; t0 += a.tg2) {
    const int tn = min(a.tg2, m - t0);
    __syncthreads();
    const int vec_per_tok = I / 4;  // float4
    for (int v = threadIdx.x; v < tn * vec_per_tok; v += kFfnThreads) {
      const int tt = v / vec_per_tok, off = v % vec_per_tok;
      const int p = Q.pairs[t0 + tt];
      reinterpret_cast<float4*>(as + (int64_t)tt * I)[off] =
          reinterpret_cast<const float4*>(a.a_buf + (int64_t)p * I)[off];
    }
    __syncthreads();
    for (int h0 = h_begin + wave * RPW; h0 < h_end; h0 += kWaves * RPW) {
      uint4 wq[RPW][NS];
      float ws[RPW][NS];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const uint4* src = reinterpret_cast<const uint4*>(W + (int64_t)(h0 + r) * rb);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int c = lane + kWave * s;
          if (c < C) {
            wq[r][s] = load_stream16(src + c);
            ws[r][s] = chunk_scale<FMT>(Ws, H, I, h0 + r, c);
          } else {
            wq[r][s] = make_uint4(0, 0, 0, 0);
            ws[r][s] = 0.0f;
          }
        }
      }
      for (int tt = 0; tt < tn; ++tt) {
        float acc[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;
        const float* at = as + (int64_t)tt * I;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int c = lane + kWave * s;
          if (c < C) {
#pragma unroll
            for (int r = 0; r < RPW; ++r)
              acc[r] = __builtin_fmaf(chunk_dot_f32<FMT>(wq[r][s], at + c * V), ws[r][s], acc[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r] = wave_sum(acc[r]);
        if (lane == 0) {
          const int p = Q.pairs[t0 + tt];
          float* dst = a.o_buf + (int64_t)p * H;
#pragma unroll
          for (int r = 0; r < RPW; ++r) dst[h0 + r] = acc[r];
        }
      }
    }
  }
}

// ---- combine ----------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(FfnArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.M * a.H) return;
  const int t = idx / a.H, h = idx % a.H;
  float y = 0.0f;
  for (int j = 0; j < a.S; ++j) {
    const int p = t * a.S + j;
    const int e = a.ids[p];
    if (e < 0 || e >= a.n_experts) continue;
    y = __builtin_fmaf(a.topk_w[p], a.o_buf[(int64_t)p * a.H + h], y);
  }
  a.y[idx] = f32_to_bf16(y);
}

template <int FMT, int NS>
hipError_t launch_gateup_ns(const FfnArgs& a, int grid, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((gateup_kernel<FMT, NS>), dim3(grid), dim3(kFfnThreads), lds, stream, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gateup(const FfnArgs& a, int ns, int grid, size_t lds, hipStream_t stream) {
  switch (ns) {
    case 1: return launch_gateup_ns<FMT, 1>(a, grid, lds, stream);
    case 2: return launch_gateup_ns<FMT, 2>(a, grid, lds, stream);
    case 3: return launch_gateup_ns<FMT, 3>(a, grid, lds, stream);
    case 4: return launch_gateup_ns<FMT, 4>(a, grid, lds, stream);
    case 5: return launch_gateup_ns<FMT, 5>(a, grid, lds, stream);
    case 6: return launch_gateup_ns<FMT, 6>(a, grid, lds, stream);
    case 7: return launch_gateup_ns<FMT, 7>(a, grid, lds, stream);
    case 8: return launch_gateup_ns<FMT, 8>(a, grid, lds, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, int NS>
hipError_t launch_down_ns(const FfnArgs& a, int grid, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((down_kernel<FMT, NS, 4>), dim3(grid), dim3(kFfnThreads), lds, stream, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_down(const FfnArgs& a, int ns, int grid, size_t lds, hipStream_t stream) {
  switch (ns) {
    case 1: return launch_down_ns<FMT, 1>(a, grid, lds, stream);
    case 2: return launch_down_ns<FMT, 2>(a, grid, lds, stream);
    case 3: return launch_down_ns<FMT, 3>(a, grid, lds, stream);
    case 4: return launch_down_ns<FMT, 4>(a, grid, lds, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

FfnPlan plan_ffn(int wfmt, int M, int S, int H, int I, int n_experts) {
  FfnPlan p;
  const int vals = (wfmt == WFMT_FP8_B128) ? 16 : 32;
  p.ns13 = (H / vals + kWave - 1) / kWave;
  p.ns2 = (I / vals + kWave - 1) / kWave;
  p.max_active = n_experts < M * S ? n_experts : M * S;
  p.ib = 2 * kWaves;  // two intermediate indices per wave
  p.items13 = I / p.ib;
  const int64_t rb2 = (wfmt == WFMT_FP8_B128) ? I : I / 2;
  // about 48 KB of W2 per down item, a multiple of 16 rows dividing H
  int hb = 16;
  while (hb < 64 && (int64_t)(2 * hb) * rb2 <= 49152 && H % (2 * hb) == 0) hb *= 2;
  p.hb = hb;
  p.items2 = H / hb;
  const int64_t lds_budget = 64 * 1024;
  int tg13 = (int)(lds_budget / (2 * (int64_t)H));
  int tg2 = (int)(lds_budget / (4 * (int64_t)I));
  const int max_tok = M * S;  // an expert can in principle hold every pair
  p.tg13 = tg13 < 1 ? 1 : (tg13 > max_tok ? max_tok : tg13);
  p.tg2 = tg2 < 1 ? 1 : (tg2 > max_tok ? max_tok : tg2);
  if (p.tg13 > M) p.tg13 = M;
  if (p.tg2 > M) p.tg2 = M;
  p.lds13 = (size_t)p.tg13 * H * 2;
  p.lds2 = (size_t)p.tg2 * I * 4;
  return p;
}

hipError_t launch_ffn(const FfnArgs& a, const FfnPlan& p, int wfmt, hipStream_t stream) {
  hipError_t err;
  FfnArgs b = a;
  b.ib = p.ib;
  b.hb = p.hb;
  b.items13 = p.items13;
  b.items2 = p.items2;
  b.tg13 = p.tg13;
  b.tg2 = p.tg2;
  const int grid13 = p.max_active * p.items13, grid2 = p.max_active * p.items2;
  if (wfmt == WFMT_FP8_B128) {
    err = launch_gateup<WFMT_FP8_B128>(b, p.ns13, grid13, p.lds13, stream);
    if (err != hipSuccess) return err;
    err = launch_down<WFMT_FP8_B128>(b, p.ns2, grid2, p.lds2, stream);
  } else {
    err = launch_gateup<WFMT_MXFP4>(b, p.ns13, grid13, p.lds13, stream);
    if (err != hipSuccess) return err;
    err = launch_down<WFMT_MXFP4>(b, p.ns2, grid2, p.lds2, stream);
  }
  if (err != hipSuccess) return err;
  const int n = a.M * a.H;
  hipLaunchKernelGGL(combine_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, b);
  return hipGetLastError();
}

}  // namespace moe
