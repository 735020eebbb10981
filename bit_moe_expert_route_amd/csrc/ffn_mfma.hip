// Expert FFN for several tokens per call on the gfx950 matrix cores.
//   d9249.github.io "glm-5-2-b300-kernel-mtp-serving", idea 3: a verify block of M tokens shares
//   one weight stream, so the expert GEMV becomes a skinny GEMM; molayo1419.me Xiaomi 1T page,
//   section 1: every active expert's weights are still read once per step.
//
// A tile is 16 rows of one active expert; its tokens (the expert's (token, slot) pairs, up to 16
// per pass) are the 16 columns of the B operand, so one load per K-step brings every token's
// activations and no token is handled in a serial pass of its own.  The workgroup's 4 waves split
// the reduction axis K into contiguous quarters and their partial 16x16 tiles are summed in LDS
// in wave order.  Weights are decoded exactly to bf16: E2M1 x 2^X with the MXFP4 block exponent
// folded into the conversion, and E4M3 as is with its 128x128 block scale applied per 128-wide K
// block to an fp32 partial.  v_mfma_f32_16x16x32_bf16 accumulates in fp32.
//
// gate/up: tile = rows i0..i0+15 of the gate and of the up matrix; a = silu(g)*u goes to the
//   workspace as two bf16 arrays, a_hi = bf16(a) and a_lo = bf16(a - a_hi), so that the down
//   projection reads an MFMA operand pair that carries a to about 16 significant bits.
// down: tile = rows h0..h0+15 of W2; B = a_hi and a_lo (two MFMAs per step); o (fp32) goes to the
//   workspace for the slot-ordered combine.
#include "ffn_common.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kTile = 16;

// K values per super-step: 4 lane groups x 16 bytes of codes.
template <int FMT>
struct Mf;
template <>
struct Mf<WFMT_MXFP4> {
  static constexpr int kKss = 128;  // 4 x 32 values
  static constexpr int kSteps = 4;  // MFMA K-steps (8 values) per lane group per super-step
};
template <>
struct Mf<WFMT_FP8_B128> {
  static constexpr int kKss = 64;   // 4 x 16 values
  static constexpr int kSteps = 2;
};

// The n-th pair (in pair order) of the masks, or -1 when there are fewer than n+1.
__device__ __forceinline__ int nth_pair(const uint64_t (&pm)[kPairRegs], int n) {
  int res = -1;
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k) {
    const int c = __popcll(pm[k]);
    if (res < 0 && n < c) {
      uint64_t m = pm[k];
      for (int i = 0; i < n; ++i) m &= m - 1;
      res = kWave * k + __builtin_ctzll(m);
    }
    n -= c;
  }
  return res;
}

__device__ __forceinline__ bf16x8 pack8(bf16x2 p0, bf16x2 p1, bf16x2 p2, bf16x2 p3) {
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16 bytes of codes -> the A operands of the super-step's K-steps (exact bf16).
template <int FMT>
__device__ __forceinline__ void decode_a(uint4 w, float scale, bf16x8 (&A)[Mf<FMT>::kSteps]) {
  opaque(w);
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  if constexpr (FMT == WFMT_MXFP4) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      A[s] = pack8(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], scale, 0),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], scale, 1),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], scale, 2),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], scale, 3));
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x2 l0, h0, l1, h1;
      fp8x4_to_bf16(d[2 * s], l0, h0);
      fp8x4_to_bf16(d[2 * s + 1], l1, h1);
      A[s] = pack8(l0, h0, l1, h1);
    }
  }
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 fma4(f32x4 t, float s, f32x4 acc) {
  f32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) r[v] = __builtin_fmaf(t[v], s, acc[v]);
  return r;
}

// Super-steps [ss0, ss1) of this wave's K quarter.  FP8 quarters are whole 128-wide blocks.
template <int FMT>
__device__ __forceinline__ void k_quarter(int K, int wave, int& ss0, int& ss1) {
  if constexpr (FMT == WFMT_FP8_B128) {
    const int nb = K / 128;
    ss0 = 2 * (nb * wave / kFfnWaves);
    ss1 = 2 * (nb * (wave + 1) / kFfnWaves);
  } else {
    const int ns = K / Mf<FMT>::kKss;
    ss0 = ns * wave / kFfnWaves;
    ss1 = ns * (wave + 1) / kFfnWaves;
  }
}

// One pass of a 16-row tile over this wave's K quarter.  wrow / wscale: this lane's A row (codes,
// scales) in each of the NM matrices (gate and up, or W2); brow: this lane's B column (bf16; a_hi
// and a_lo when NB == 2).  Returns the partial tiles in D[NM].
template <int FMT, int NM, int NB>
__device__ __forceinline__ void tile_pass(const uint8_t* const (&wrow)[NM],
                                          const void* const (&wscale)[NM],
                                          const uint16_t* const (&brow)[NB], bool colv, int grp,
                                          int ss0, int ss1, f32x4 (&D)[NM]) {
  constexpr int KSS = Mf<FMT>::kKss, NST = Mf<FMT>::kSteps;
  constexpr int U = 4;  // super-steps of loads in flight per iteration
#pragma unroll
  for (int mi = 0; mi < NM; ++mi) D[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 T[NM];  // FP8: partial of the current 128-wide K block
#pragma unroll
  for (int mi = 0; mi < NM; ++mi) T[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = ss0; s0 < ss1; s0 += U) {
    uint4 w[U][NM];
    uint32_t sc[U][NM];
    uint4 x[U][NB][NST];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ss = (s0 + u < ss1) ? s0 + u : ss1 - 1;  // clamped: loads stay unconditional
      const int koff = ss * KSS + grp * (KSS / 4);       // first K value of this lane group
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
        if constexpr (FMT == WFMT_MXFP4) {
          w[u][mi] = load_stream16(wrow[mi] + koff / 2);
          sc[u][mi] = reinterpret_cast<const uint8_t*>(wscale[mi])[koff / 32];
        } else {
          w[u][mi] = load_stream16(wrow[mi] + koff);
          sc[u][mi] = reinterpret_cast<const uint32_t*>(wscale[mi])[koff / 128];
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int st = 0; st < NST; ++st)
          x[u][b][st] = *reinterpret_cast<const uint4*>(brow[b] + koff + 8 * st);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < ss1) {
        const int ss = s0 + u;
        bf16x8 B[NB][NST];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int st = 0; st < NST; ++st) {
            const uint4 v = x[u][b][st];
            B[b][st] = as_bf16x8(colv ? v : make_uint4(0, 0, 0, 0));
          }
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
          bf16x8 A[NST];
          if constexpr (FMT == WFMT_MXFP4) {
            decode_a<FMT>(w[u][mi], e8m0_to_f32(sc[u][mi]), A);
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
              for (int b = 0; b < NB; ++b) D[mi] = mfma(A[st], B[b][st], D[mi]);
          } else {
            decode_a<FMT>(w[u][mi], 1.0f, A);
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
              for (int b = 0; b < NB; ++b) T[mi] = mfma(A[st], B[b][st], T[mi]);
            if (ss & 1) {  // end of a 128-wide block: apply its scale
              D[mi] = fma4(T[mi], __uint_as_float(sc[u][mi]), D[mi]);
              T[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
      }
    }
  }
}

// Sum of the 4 waves' partial tiles, in wave order, into wave 0.  red: [3][NM][64] f32x4.
template <int NM>
__device__ __forceinline__ void reduce_waves(f32x4 (&D)[NM], f32x4* red, int wave, int lane) {
  if (wave > 0) {
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) red[((wave - 1) * NM + mi) * kWave + lane] = D[mi];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < kFfnWaves; ++w)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
        const f32x4 o = red[((w - 1) * NM + mi) * kWave + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) D[mi][v] += o[v];
      }
  }
}

// Tiles of the expert-major tile list for this workgroup: [T*b/G, T*(b+1)/G).
__device__ __forceinline__ void wg_tiles(int T, int& t0, int& t1) {
  t0 = (int)((int64_t)T * blockIdx.x / gridDim.x);
  t1 = (int)((int64_t)T * (blockIdx.x + 1) / gridDim.x);
}

template <int FMT>
__global__ __launch_bounds__(kFfnThreads) void gateup_mfma_kernel(FfnArgs a) {
  __shared__ QueueLds QL;
  __shared__ f32x4 red[(kFfnWaves - 1) * 2 * kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int H = a.H, I = a.I, S = a.S;
  const int col = lane % kTile, grp = lane / kTile;
  int ss0, ss1;
  k_quarter<FMT>(H, wave, ss0, ss1);
  const int tpe = I / kTile;
  int t0, t1;
  wg_tiles(Q.n_active * tpe, t0, t1);
  const int64_t rb = Fmt<FMT>::row_bytes(H);
  uint16_t* a_hi = reinterpret_cast<uint16_t*>(a.a_buf);
  uint16_t* a_lo = a_hi + (int64_t)a.M * S * I;
  for (int t = t0; t < t1; ++t) {
    const int q = t / tpe, i0 = (t % tpe) * kTile;
    const int e = wave_queue_expert(Q, q);
    uint64_t pm[kPairRegs];
    wave_queue_pairs(Q, q, pm);
    int m = 0;
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) m += __popcll(pm[k]);
    const int p_first = first_pair(pm);
    const uint8_t* W = a.w13 + (int64_t)e * 2 * I * rb;
    const void* Ws = scale_ptr<FMT>(a.w13s, (int64_t)e * scale_elems<FMT>(2 * I, H));
    const int rg = i0 + col, ru = I + i0 + col;  // this lane's A rows
    const uint8_t* const wrow[2] = {W + rg * rb, W + ru * rb};
    const void* wscale[2];
    if constexpr (FMT == WFMT_MXFP4) {
      wscale[0] = reinterpret_cast<const uint8_t*>(Ws) + (int64_t)rg * (H / 32);
      wscale[1] = reinterpret_cast<const uint8_t*>(Ws) + (int64_t)ru * (H / 32);
    } else {
      wscale[0] = reinterpret_cast<const float*>(Ws) + (int64_t)(rg >> 7) * (H >> 7);
      wscale[1] = reinterpret_cast<const float*>(Ws) + (int64_t)(ru >> 7) * (H >> 7);
    }
    for (int pg = 0; pg < m; pg += kTile) {
      const int p = nth_pair(pm, pg + col);
      const bool colv = p >= 0;
      const uint16_t* const xrow[1] = {a.x + (int64_t)((colv ? p : p_first) / S) * H};
      f32x4 D[2];
      tile_pass<FMT, 2, 1>(wrow, wscale, xrow, colv, grp, ss0, ss1, D);
      reduce_waves<2>(D, red, wave, lane);
      if (wave == 0 && colv) {
        // lane (col, grp) holds rows i0 + 4*grp + v of column col
        uint32_t hi[2], lo[2];
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2) {
          uint32_t h2 = 0, l2 = 0;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int v = 2 * v2 + h;
            const float g = D[0][v], u = D[1][v];
            const float av = (g / (1.0f + __expf(-g))) * u;
            const uint16_t hb = f32_to_bf16(av);
            const uint16_t lb = f32_to_bf16(av - bf16_to_f32(hb));
            h2 |= (uint32_t)hb << (16 * h);
            l2 |= (uint32_t)lb << (16 * h);
          }
          hi[v2] = h2;
          lo[v2] = l2;
        }
        const int64_t off = (int64_t)p * I + i0 + 4 * grp;
        *reinterpret_cast<uint2*>(a_hi + off) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2*>(a_lo + off) = make_uint2(lo[0], lo[1]);
      }
      __syncthreads();  // red is reused by the next tile
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kFfnThreads) void down_mfma_kernel(FfnArgs a) {
  __shared__ QueueLds QL;
  __shared__ f32x4 red[(kFfnWaves - 1) * kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int H = a.H, I = a.I, S = a.S;
  const int col = lane % kTile, grp = lane / kTile;
  int ss0, ss1;
  k_quarter<FMT>(I, wave, ss0, ss1);
  const int tpe = H / kTile;
  int t0, t1;
  wg_tiles(Q.n_active * tpe, t0, t1);
  const int64_t rb = Fmt<FMT>::row_bytes(I);
  const uint16_t* a_hi = reinterpret_cast<const uint16_t*>(a.a_buf);
  const uint16_t* a_lo = a_hi + (int64_t)a.M * S * I;
  for (int t = t0; t < t1; ++t) {
    const int q = t / tpe, h0 = (t % tpe) * kTile;
    const int e = wave_queue_expert(Q, q);
    uint64_t pm[kPairRegs];
    wave_queue_pairs(Q, q, pm);
    int m = 0;
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) m += __popcll(pm[k]);
    const int p_first = first_pair(pm);
    const uint8_t* W = a.w2 + (int64_t)e * H * rb;
    const void* Ws = scale_ptr<FMT>(a.w2s, (int64_t)e * scale_elems<FMT>(H, I));
    const int r = h0 + col;
    const uint8_t* const wrow[1] = {W + r * rb};
    const void* wscale[1];
    if constexpr (FMT == WFMT_MXFP4)
      wscale[0] = reinterpret_cast<const uint8_t*>(Ws) + (int64_t)r * (I / 32);
    else
      wscale[0] = reinterpret_cast<const float*>(Ws) + (int64_t)(r >> 7) * (I >> 7);
    for (int pg = 0; pg < m; pg += kTile) {
      const int p = nth_pair(pm, pg + col);
      const bool colv = p >= 0;
      const int pc = colv ? p : p_first;
      const uint16_t* const brow[2] = {a_hi + (int64_t)pc * I, a_lo + (int64_t)pc * I};
      f32x4 D[1];
      tile_pass<FMT, 1, 2>(wrow, wscale, brow, colv, grp, ss0, ss1, D);
      reduce_waves<1>(D, red, wave, lane);
      if (wave == 0 && colv)
        *reinterpret_cast<f32x4*>(a.o_buf + (int64_t)p * H + h0 + 4 * grp) = D[0];
      __syncthreads();
    }
  }
}

template <typename K>
hipError_t launch_resident(K kern, int* grid, const FfnArgs& a, hipStream_t stream) {
  hipError_t err = resident_grid(kern, grid);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(*grid), dim3(kFfnThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_mfma(const FfnArgs& a, int wfmt, hipStream_t stream) {
  static int g_fp8 = 0, g_mx = 0;
  return wfmt == WFMT_FP8_B128
             ? launch_resident(gateup_mfma_kernel<WFMT_FP8_B128>, &g_fp8, a, stream)
             : launch_resident(gateup_mfma_kernel<WFMT_MXFP4>, &g_mx, a, stream);
}

hipError_t launch_down_mfma(const FfnArgs& a, int wfmt, hipStream_t stream) {
  static int g_fp8 = 0, g_mx = 0;
  return wfmt == WFMT_FP8_B128
             ? launch_resident(down_mfma_kernel<WFMT_FP8_B128>, &g_fp8, a, stream)
             : launch_resident(down_mfma_kernel<WFMT_MXFP4>, &g_mx, a, stream);
}

}  // namespace moe
