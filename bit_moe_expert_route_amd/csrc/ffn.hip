// Expert FFN decode in one persistent launch: stream each active expert's packed W13 and W2
// once, SwiGLU in between, weighted combine in slot order.
//   molayo1419.me Xiaomi 1T page, section 1: decode reads every active weight from HBM once per
//   step and is bound by bandwidth; section 2: expert FFN weights in MXFP4.
//   d9249.github.io "glm-5-2-b300-kernel-mtp-serving", table under "what it solves" and idea 1:
//   a batch-1 expert GEMM needs many long concurrent memory streams to approach peak bandwidth;
//   idea 2: scale handling must not stall the load pipeline; idea 3: a verify block of M tokens
//   shares one weight stream.
//   blogs.novita.ai "Optimizing GLM4-MoE for production", section 1: the shared expert runs as
//   one more slot of the same fused MoE.
//
// Structure: three launches, stream-ordered (a kernel boundary is the cheapest device-wide
// barrier here: device-scope atomics on a few shared counters and release fences cost more
// than a launch).
//   gate/up : persistent grid; unit = one intermediate index i of one active expert (rows
//             gate_i and up_i).  Each wave owns a contiguous range of units, so it streams long
//             runs of consecutive rows; lanes cover the 16-byte chunks c = lane + 64*s of a row,
//             which keeps each lane's slice of the first token's activations in registers for
//             the whole run; a = silu(g)*u goes to the workspace.
//   down    : persistent grid; unit = RPW rows of W2 of one active expert, same lane layout,
//             a in registers per expert; o goes to the workspace.
//   combine : y[t][h] = sum_j w[t][j] * o[t][j][h] in slot order, rounded to bf16.
// Every wave of the first two derives the expert-sorted queue (distinct experts ascending,
// each with its (token, slot) pairs) from the routing ids, without workgroup barriers.
#include <type_traits>

#include "act_quant.h"
#include "ffn_common.h"
#include "route_select.h"

namespace moe {
namespace {

// Partial dot product of one 16-byte weight chunk with bf16 activations (kXWords pairs).
// The chunk passes through opaque() so its decode stays inside the caller's per-token loop.
template <int FMT>
__device__ __forceinline__ float chunk_dot_bf16(uint4 wq, const uint32_t* xw) {
  opaque(wq);
  const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
  float acc = 0.0f;
  if constexpr (FMT == WFMT_FP8_B128) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x2 lo, hi;
      fp8x4_to_bf16(ww[j], lo, hi);
      acc = dot2(lo, as_bf16x2(xw[2 * j]), acc);
      acc = dot2(hi, as_bf16x2(xw[2 * j + 1]), acc);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x2 wb[4];
      fp4x8_to_bf16(ww[j], wb);
#pragma unroll
      for (int b = 0; b < 4; ++b) acc = dot2(wb[b], as_bf16x2(xw[4 * j + b]), acc);
    }
  }
  return acc;
}

// Partial dot product of one 16-byte weight chunk with fp32 activations (kVals floats).
template <int FMT>
__device__ __forceinline__ float chunk_dot_f32(uint4 wq, const float* av) {
  opaque(wq);
  const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
  float acc = 0.0f;
  if constexpr (FMT == WFMT_FP8_B128) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 lo = fp8x2_to_f32<false>(ww[j]), hi = fp8x2_to_f32<true>(ww[j]);
      acc = __builtin_fmaf(lo.x, av[4 * j], acc);
      acc = __builtin_fmaf(lo.y, av[4 * j + 1], acc);
      acc = __builtin_fmaf(hi.x, av[4 * j + 2], acc);
      acc = __builtin_fmaf(hi.y, av[4 * j + 3], acc);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 p0 = fp4x2_to_f32<0>(ww[j]), p1 = fp4x2_to_f32<1>(ww[j]);
      const f32x2 p2 = fp4x2_to_f32<2>(ww[j]), p3 = fp4x2_to_f32<3>(ww[j]);
      acc = __builtin_fmaf(p0.x, av[8 * j], acc);
      acc = __builtin_fmaf(p0.y, av[8 * j + 1], acc);
      acc = __builtin_fmaf(p1.x, av[8 * j + 2], acc);
      acc = __builtin_fmaf(p1.y, av[8 * j + 3], acc);
      acc = __builtin_fmaf(p2.x, av[8 * j + 4], acc);
      acc = __builtin_fmaf(p2.y, av[8 * j + 5], acc);
      acc = __builtin_fmaf(p3.x, av[8 * j + 6], acc);
      acc = __builtin_fmaf(p3.y, av[8 * j + 7], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return (g / (1.0f + __expf(-g))) * u;
}

// gate/up + SwiGLU for one token, software-pipelined.  Wave g takes the units
// [U*g/NW, U*(g+1)/NW) of the expert-major list (unit = intermediate index i of one active
// expert: rows gate_i and up_i).  The next unit's loads are always in flight while the current
// unit is reduced, with the same loads every step (a prefetch past the wave's last unit reads
// the current expert's first chunk and is discarded), so a wave's time follows its bytes rather
// than its count of load batches.  The token's activations stay in registers.  The reduced
// values collect in one register across lanes (lane j holds the wave's j-th value) and are
// stored 64 at a time, which keeps stores out of the load pipeline.
template <int FMT, int NS>
__device__ void gateup_one_token(const FfnArgs& a, const WaveQueue& Q, int gw, int NW) {
  constexpr int V = Fmt<FMT>::kVals;
  constexpr int XW = Fmt<FMT>::kXWords;
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I;
  const int C = H / V;
  const int64_t rb = Fmt<FMT>::row_bytes(H);
  const int U = Q.n_active * I;
  const int u0 = (int)((int64_t)U * gw / NW), u1 = (int)((int64_t)U * (gw + 1) / NW);
  if (u0 >= u1) return;
  int cs[NS];
  bool cv[NS];
#pragma unroll
  for (int sI = 0; sI < NS; ++sI) {
    const int c = lane + kWave * sI;
    cv[sI] = c < C;
    cs[sI] = cv[sI] ? c : C - 1;
  }
  uint32_t xr[NS][XW];
  {
    const uint32_t* xs = reinterpret_cast<const uint32_t*>(a.x);
#pragma unroll
    for (int sI = 0; sI < NS; ++sI)
#pragma unroll
      for (int k4 = 0; k4 < XW / 4; ++k4) {
        const uint4 v = reinterpret_cast<const uint4*>(xs + (int64_t)cs[sI] * XW)[k4];
        xr[sI][4 * k4] = v.x;
        xr[sI][4 * k4 + 1] = v.y;
        xr[sI][4 * k4 + 2] = v.z;
        xr[sI][4 * k4 + 3] = v.w;
      }
  }
  struct Buf {
    uint4 w[2][NS];      // [gate, up][chunk]
    uint32_t sc[2][NS];  // raw block scales
  };
  // load cursor: rank lq, index li, expert le of the next unit to load
  int lq = u0 / I, li = u0 - lq * I;
  int le = wave_queue_expert(Q, lq);
  auto load = [&](Buf& b, bool valid) {
    // a discarded prefetch reads the expert's first row: every offset is and-ed with a
    // wave-uniform mask (a select here would become a branch around each load)
    int vm = __builtin_amdgcn_readfirstlane(valid ? -1 : 0);
    opaque(vm);
    const uint8_t* W = a.w13 + (int64_t)le * 2 * I * rb;
    const void* Ws = scale_ptr<FMT>(a.w13s, (int64_t)le * scale_elems<FMT>(2 * I, H));
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = (r * I + li) & vm;
      const uint8_t* src = W + (int64_t)row * rb;
#pragma unroll
      for (int sI = 0; sI < NS; ++sI) {
        b.w[r][sI] = load_stream16(src + (int64_t)(cs[sI] & vm) * 16);
        b.sc[r][sI] = scale_raw<FMT>(Ws, H, row, cs[sI] & vm);
      }
    }
  };
  auto advance = [&]() {
    if (++li == I) {
      li = 0;
      ++lq;
      if (lq < Q.n_active) le = wave_queue_expert(Q, lq);
    }
  };
  int cq = -1;  // rank whose pairs are in pm
  uint64_t pm[kPairRegs] = {};
  float outv = 0.0f;
  int64_t outi = 0;
  int nout = 0;
  auto compute = [&](const Buf& b, int u) {
    const int q = u / I, i = u - q * I;
    if (q != cq) {
      cq = q;
      wave_queue_pairs(Q, q, pm);
    }
    float g = 0.0f, up = 0.0f;
#pragma unroll
    for (int sI = 0; sI < NS; ++sI) {
      const float ng = __builtin_fmaf(chunk_dot_bf16<FMT>(b.w[0][sI], xr[sI]),
                                      scale_value<FMT>(b.sc[0][sI]), g);
      const float nu = __builtin_fmaf(chunk_dot_bf16<FMT>(b.w[1][sI], xr[sI]),
                                      scale_value<FMT>(b.sc[1][sI]), up);
      g = cv[sI] ? ng : g;
      up = cv[sI] ? nu : up;
    }
    g = wave_sum_to_last(g);
    up = wave_sum_to_last(up);
    const float val =
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(silu_mul(g, up)), kWave - 1));
    // one value per pair of the expert (several only for a duplicated id)
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) {
      for (uint64_t m = pm[k]; m; m &= m - 1) {
        const int p = kWave * k + __builtin_ctzll(m);
        outv = lane == nout ? val : outv;
        outi = lane == nout ? (int64_t)p * I + i : outi;
        if (++nout == kWave) {
          a.a_buf[outi] = outv;
          nout = 0;
        }
      }
    }
  };
  Buf A, B;
  load(A, true);
  advance();
  for (int u = u0; u < u1; u += 2) {
    const bool has_b = u + 1 < u1;
    load(B, has_b);
    if (has_b) advance();
    compute(A, u);
    const bool has_a = u + 2 < u1;
    load(A, has_a);
    if (has_a) advance();
    if (has_b) compute(B, u + 1);
  }
  if (lane < nout) a.a_buf[outi] = outv;
}

// gate/up + SwiGLU in batches.  Each iteration takes up to two consecutive units of the same
// expert (four rows, 4*NS loads in flight per lane) and runs every (token, slot) pair of that
// expert over them; the expert's first token keeps its activations in registers, further
// tokens read theirs from L2.  Part `part` of `nparts` takes the units of a cost-weighted split
// (a unit costs one pass per pair; with one token, a plain split).
// - DYN = false: the parts are waves, each walking its own range, two units per iteration.
// - DYN = true: the parts are workgroups (one per CU); a workgroup's waves take UPG units at a
//   time from its LDS counter `next`, so they finish together.  With UPG = 2 the part
//   boundaries sit at even units, so a pair of units never straddles two experts (I is even).
// A8: W8A8 with one token.  The caller has loaded the token's activations into xv; right after
// issuing its first unit's weight loads (or finding it has none) each wave quantizes its share
// into xl and meets the others at the workgroup barrier, so the quantization overlaps the first
// weight loads.  Every pair then belongs to the one token and takes its activations from
// registers.
// AW: W8A8 with several tokens: x and its block scales were quantized into the workspace by a
// pass of their own (xq, x_scales); the first token's scales are kept with its chunks, a further
// token's are read with its chunk.
template <int FMT, int NS, int UPG, bool DYN, bool A8, bool AW = false>
__device__ __forceinline__ void gateup_tokens(const FfnArgs& a, const WaveQueue& Q, int* cnt,
                                              int* next, int part, int nparts,
                                              ActLds* xl = nullptr,
                                              const ActX<kFfnThreads, (NS + 1) / 2>* xv = nullptr) {
  static_assert(UPG == 1 || UPG == 2, "one or two units per iteration");
  static_assert(!A8 || FMT == WFMT_FP8_B128, "W8A8 takes FP8 weights");
  constexpr int V = Fmt<FMT>::kVals;
  constexpr int XW = Fmt<FMT>::kXWords;
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I, S = a.S;
  const int C = H / V;
  const int64_t rb = Fmt<FMT>::row_bytes(H);
  // one token: every unit costs the same, plain split; else the cost-weighted split
  constexpr int kAlign = (DYN && UPG == 2) ? ~1 : ~0;
  int u0, u1;
  if (a.M == 1) {
    const int U = Q.n_active * I;
    u0 = (int)((int64_t)U * part / nparts) & kAlign;
    u1 = (int)((int64_t)U * (part + 1) / nparts) & kAlign;
  } else {
    WaveBalance B;
    wave_balance_build(B, Q, cnt, I, kUnitCost, kPairCost);
    u0 = wave_balance_unit(B, (int64_t)B.total * part / nparts) & kAlign;
    u1 = wave_balance_unit(B, (int64_t)B.total * (part + 1) / nparts) & kAlign;
  }
  if constexpr (DYN) {
    if (threadIdx.x == 0) *next = u0;
    __syncthreads();
  }
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(next, UPG);
    return __builtin_amdgcn_readfirstlane(v);
  };
  // lane chunks c_s = lane + 64*s, clamped into the row so every load is in bounds; clamped
  // (invalid) chunks are masked out of the sums with selects
  int cs[NS];
  bool cv[NS];
#pragma unroll
  for (int sI = 0; sI < NS; ++sI) {
    const int c = lane + kWave * sI;
    cv[sI] = c < C;
    cs[sI] = cv[sI] ? c : C - 1;
  }
  auto load_x_chunk = [&](const uint32_t* xs, int sI, uint32_t (&dst)[XW]) {
#pragma unroll
    for (int k4 = 0; k4 < XW / 4; ++k4) {
      const uint4 v = reinterpret_cast<const uint4*>(xs + (int64_t)cs[sI] * XW)[k4];
      dst[4 * k4] = v.x; dst[4 * k4 + 1] = v.y; dst[4 * k4 + 2] = v.z; dst[4 * k4 + 3] = v.w;
    }
  };
  uint32_t xr[NS][XW];  // first token of the current expert, this lane's chunks
  float xsc[NS];        // A8: their block scales
  bool staged = !A8;    // A8: this wave has quantized its share and passed the barrier
  uint64_t pm[kPairRegs] = {};
  int cur_q = -1, e = 0, p0 = 0;
  for (int u = DYN ? grab() : u0; u < u1;) {
    const int q = u / I, i = u % I;
    if (q != cur_q) e = wave_queue_expert(Q, q);
    const int nu = (UPG == 2 && u + 1 < u1 && i + 1 < I) ? 2 : 1;  // units this iteration
    const uint8_t* W = a.w13 + (int64_t)e * 2 * I * rb;
    const void* Ws = scale_ptr<FMT>(a.w13s, (int64_t)e * scale_elems<FMT>(2 * I, H));
    uint4 w[2][2][NS];      // [unit][gate, up][chunk]
    uint32_t sc[2][2][NS];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (d < nu) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = r * I + i + d;
          const uint8_t* src = W + (int64_t)row * rb;
#pragma unroll
          for (int sI = 0; sI < NS; ++sI) {
            w[d][r][sI] = load_stream16(src + (int64_t)cs[sI] * 16);
            sc[d][r][sI] = scale_raw<FMT>(Ws, H, row, cs[sI]);
          }
        }
      }
    }
    if constexpr (A8) {
      if (!staged) {
        act_x_quant_store(*xv, H, *xl);
        __syncthreads();
        staged = true;
      }
    }
    if (q != cur_q) {
      cur_q = q;
      wave_queue_pairs(Q, q, pm);
      p0 = first_pair(pm);
      if constexpr (A8) {
#pragma unroll
        for (int sI = 0; sI < NS; ++sI) {
          load_x_chunk(xl->xq, sI, xr[sI]);
          xsc[sI] = xl->xs[cs[sI] >> 3];
        }
      } else {
        const uint16_t* xsrc = AW ? a.xq : a.x;
        const uint32_t* xs = reinterpret_cast<const uint32_t*>(xsrc + (int64_t)(p0 / S) * H);
#pragma unroll
        for (int sI = 0; sI < NS; ++sI) {
          load_x_chunk(xs, sI, xr[sI]);
          if constexpr (AW) xsc[sI] = a.x_scales[(int64_t)(p0 / S) * (H >> 7) + (cs[sI] >> 3)];
        }
      }
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (d < nu) {
        // every pair of the expert, in pair order
#pragma unroll
        for (int k = 0; k < kPairRegs; ++k) {
          for (uint64_t m = pm[k]; m; m &= m - 1) {
            const int p = kWave * k + __builtin_ctzll(m);
            float g = 0.0f, up = 0.0f;
            if (A8 || p == p0) {
#pragma unroll
              for (int sI = 0; sI < NS; ++sI) {
                float sg = scale_value<FMT>(sc[d][0][sI]), su = scale_value<FMT>(sc[d][1][sI]);
                if constexpr (A8 || AW) { sg *= xsc[sI]; su *= xsc[sI]; }
                const float ng = __builtin_fmaf(chunk_dot_bf16<FMT>(w[d][0][sI], xr[sI]), sg, g);
                const float nu2 = __builtin_fmaf(chunk_dot_bf16<FMT>(w[d][1][sI], xr[sI]), su, up);
                g = cv[sI] ? ng : g;
                up = cv[sI] ? nu2 : up;
              }
            } else {
              // further tokens of the expert: activations chunk by chunk from L2
              const uint16_t* xsrc = AW ? a.xq : a.x;
              const uint32_t* xs = reinterpret_cast<const uint32_t*>(xsrc + (int64_t)(p / S) * H);
#pragma unroll
              for (int sI = 0; sI < NS; ++sI) {
                uint32_t xt[XW];
                load_x_chunk(xs, sI, xt);
                float sg = scale_value<FMT>(sc[d][0][sI]);
                float su = scale_value<FMT>(sc[d][1][sI]);
                if constexpr (AW) {
                  const float st = a.x_scales[(int64_t)(p / S) * (H >> 7) + (cs[sI] >> 3)];
                  sg *= st;
                  su *= st;
                }
                const float ng = __builtin_fmaf(chunk_dot_bf16<FMT>(w[d][0][sI], xt), sg, g);
                const float nu2 = __builtin_fmaf(chunk_dot_bf16<FMT>(w[d][1][sI], xt), su, up);
                g = cv[sI] ? ng : g;
                up = cv[sI] ? nu2 : up;
              }
            }
            g = wave_sum_to_last(g);
            up = wave_sum_to_last(up);
            if (lane == kWave - 1) a.a_buf[(int64_t)p * I + i + d] = silu_mul(g, up);
          }
        }
      }
    }
    u = DYN ? grab() : u + nu;
  }
  if constexpr (A8) {
    if (!staged) {  // no units: still quantize this wave's share and meet the barrier once
      act_x_quant_store(*xv, H, *xl);
      __syncthreads();
    }
  }
}

// One token with MXFP4 weights takes the pipelined body: half the bytes per row of FP8 make a
// wave's batches short, and batch count (not bytes) set its time (measured: 33.3 -> 30.3 us on
// the 1T-class gate/up).  With FP8 weights the two bodies measured the same.
// AW: W8A8 with several tokens at chunk counts whose workgroup-per-CU form would spill (x and
// its scales quantized into the workspace beforehand).
template <int FMT, int NS, bool AW = false>
__device__ __forceinline__ void gateup_body(const FfnArgs& a, const WaveQueue& Q, int* cnt,
                                            int gw, int NW) {
  if (FMT == WFMT_MXFP4 && a.M == 1)
    gateup_one_token<FMT, NS>(a, Q, gw, NW);
  else
    gateup_tokens<FMT, NS, 2, false, false, AW>(a, Q, cnt, nullptr, gw, NW);
}

// gate/up of the experts the routing ids in global memory name.
// The work queue of a gate/up wave: from the routing ids, or (one token, logits set) from the
// wave's own selection over the logits, whose result the grid's first wave publishes.  The
// selection's register arrays are sized by the experts per lane (3, 6 or 16).
__device__ __forceinline__ void gateup_queue(const FfnArgs& a, WaveQueue& Q, uint32_t* bits,
                                             int* base) {
  if (a.logits == nullptr) {
    wave_queue_build(Q, bits, base, a.ids, a.M * a.S, a.n_experts);
    return;
  }
  const int lane = threadIdx.x % kWave;
  const int per = (a.E_routed + kWave - 1) / kWave;
  const int has_shared = a.S - a.k_routed;
  // only the publishing wave needs the weights (the queue needs the ids alone)
  const bool pub = blockIdx.x == 0 && threadIdx.x < kWave;
  int id;
  float w;
  if (per <= 3)
    wave_select<3>(a.logits, a.E_routed, a.k_routed, has_shared, id, w, pub);
  else if (per <= 6)
    wave_select<6>(a.logits, a.E_routed, a.k_routed, has_shared, id, w, pub);
  else
    wave_select<(kMaxExperts + kWave - 2) / kWave>(a.logits, a.E_routed, a.k_routed, has_shared,
                                                   id, w, pub);
  if (pub && lane < a.S) {
    a.ids_out[lane] = id;
    a.w_out[lane] = w;
  }
  int v[kPairRegs];
  v[0] = id;
#pragma unroll
  for (int k = 1; k < kPairRegs; ++k) v[k] = -1;
  wave_queue_from(Q, bits, base, v, a.S, a.n_experts);
}

// A8 (one token): the workgroup stages the token's quantized activations in LDS.  AW: several
// W8A8 tokens read from the workspace (per-wave split).
template <int FMT, int NS, bool A8, bool AW = false>
__global__ __launch_bounds__(kFfnThreads) void gateup_kernel(FfnArgs a) {
  static_assert(!(A8 && AW), "one token or several");
  __shared__ QueueLds QL;
  __shared__ typename std::conditional<A8, ActLds, char>::type XL;
  // NS chunks of 16 values per lane cover H, so (NS + 1) / 2 pieces of 8 per thread do
  typename std::conditional<A8, ActX<kFfnThreads, (NS + 1) / 2>, char>::type XV;
  if constexpr (A8) act_x_load(a.x, a.H, XV);
  const int wave = threadIdx.x / kWave;
  WaveQueue Q;
  gateup_queue(a, Q, QL.bits[wave], QL.base[wave]);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  if constexpr (A8) {
    gateup_tokens<FMT, NS, 2, false, true>(a, Q, QL.cnt[wave], nullptr,
                                           blockIdx.x * kFfnWaves + wave, gridDim.x * kFfnWaves,
                                           &XL, &XV);
  } else {
    gateup_body<FMT, NS, AW>(a, Q, QL.cnt[wave], blockIdx.x * kFfnWaves + wave,
                             gridDim.x * kFfnWaves);
  }
}

// gate/up with several tokens: one workgroup of TPB threads per CU whose waves take UPG units
// at a time from an LDS counter.  One unit per step when the registers allow three waves per
// SIMD, else two units per step at two waves per SIMD.
template <int FMT, int NS, int UPG, int TPB, bool AW>
__global__ __launch_bounds__(TPB) void gateup_cu_kernel(FfnArgs a) {
  constexpr int NWV = TPB / kWave;
  __shared__ QueueLdsT<NWV> QL;
  const int wave = threadIdx.x / kWave;
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  gateup_tokens<FMT, NS, UPG, true, false, AW>(a, Q, QL.cnt[wave], &QL.next, blockIdx.x,
                                               gridDim.x);
}

// down projection: each iteration takes RPW2 consecutive rows of one expert.  DYN = false:
// every wave walks its own range of an equal (one token) or cost-weighted split.  DYN = true:
// one workgroup of TPB threads per CU takes such a range and its waves take its units one at a
// time from an LDS counter (as in the multi-token gate/up).
// AW: W8A8 with several tokens: a_buf already holds the quantized values and a_scales their
// block scales (a pass of their own).
template <int FMT, int NS2, int RPW2, bool DYN, int TPB, bool A8, bool AW = false>
__global__ __launch_bounds__(TPB) void down_kernel(FfnArgs a) {
  static_assert(!A8 || FMT == WFMT_FP8_B128, "W8A8 takes FP8 weights");
  constexpr int NWV = TPB / kWave;
  __shared__ QueueLdsT<NWV> QL;
  constexpr int V = Fmt<FMT>::kVals;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int H = a.H, I = a.I;
  const int part = DYN ? (int)blockIdx.x : (int)blockIdx.x * NWV + wave;
  const int nparts = DYN ? (int)gridDim.x : (int)gridDim.x * NWV;
  const int C2 = I / V;
  const int64_t rb2 = Fmt<FMT>::row_bytes(I);
  const int units_per_expert = H / RPW2;
  int v0, v1;
  if (a.M == 1) {
    const int U = Q.n_active * units_per_expert;
    v0 = (int)((int64_t)U * part / nparts);
    v1 = (int)((int64_t)U * (part + 1) / nparts);
  } else {
    WaveBalance B;
    wave_balance_build(B, Q, QL.cnt[wave], units_per_expert, kUnitCost, kPairCost);
    v0 = wave_balance_unit(B, (int64_t)B.total * part / nparts);
    v1 = wave_balance_unit(B, (int64_t)B.total * (part + 1) / nparts);
  }
  if constexpr (DYN) {
    if (threadIdx.x == 0) QL.next = v0;
    __syncthreads();
  }
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&QL.next, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int cs[NS2];
  bool cv[NS2];
#pragma unroll
  for (int sI = 0; sI < NS2; ++sI) {
    const int c = lane + kWave * sI;
    cv[sI] = c < C2;
    cs[sI] = cv[sI] ? c : C2 - 1;
  }
  auto load_a_chunk = [&](const float* as, int sI, float (&dst)[V]) {
#pragma unroll
    for (int k4 = 0; k4 < V / 4; ++k4) {
      const float4 f = reinterpret_cast<const float4*>(as + (int64_t)cs[sI] * V)[k4];
      dst[4 * k4] = f.x; dst[4 * k4 + 1] = f.y; dst[4 * k4 + 2] = f.z; dst[4 * k4 + 3] = f.w;
    }
  };
  float ar[NS2][V];  // first token of the current expert, this lane's chunks of a
  // A8 (one token): their block scales (8 chunks = 8 lanes per block, I % 128 == 0).  With one
  // token every pair of an expert has the same a (same input, weights and arithmetic), so the
  // first pair's quantized a serves them all.
  float asc[NS2];
  uint64_t pm[kPairRegs] = {};
  int cur_q = -1, e = 0, p0 = 0;
  for (int v = DYN ? grab() : v0; v < v1; v = DYN ? grab() : v + 1) {
    const int q = v / units_per_expert, h0 = (v % units_per_expert) * RPW2;
    const bool fresh = q != cur_q;
    if (fresh) e = wave_queue_expert(Q, q);
    // A8: the new expert's a is loaded before the weights (see down_flat_kernel)
    auto load_first_a = [&]() {
      cur_q = q;
      wave_queue_pairs(Q, q, pm);
      p0 = first_pair(pm);
      const float* as = a.a_buf + (int64_t)p0 * I;
#pragma unroll
      for (int sI = 0; sI < NS2; ++sI) load_a_chunk(as, sI, ar[sI]);
    };
    if constexpr (A8) {
      if (fresh) load_first_a();
    }
    const uint8_t* W = a.w2 + (int64_t)e * H * rb2;
    const void* Ws = scale_ptr<FMT>(a.w2s, (int64_t)e * scale_elems<FMT>(H, I));
    uint4 w[RPW2][NS2];
    uint32_t sc[RPW2][NS2];
#pragma unroll
    for (int r = 0; r < RPW2; ++r) {
      const uint8_t* src = W + (int64_t)(h0 + r) * rb2;
#pragma unroll
      for (int sI = 0; sI < NS2; ++sI) {
        w[r][sI] = load_stream16(src + (int64_t)cs[sI] * 16);
        sc[r][sI] = scale_raw<FMT>(Ws, I, h0 + r, cs[sI]);
      }
    }
    if (fresh) {
      if constexpr (A8) {
#pragma unroll
        for (int sI = 0; sI < NS2; ++sI) asc[sI] = act_quant_f32<8>(ar[sI]);
      } else {
        load_first_a();
        if constexpr (AW) {
#pragma unroll
          for (int sI = 0; sI < NS2; ++sI)
            asc[sI] = a.a_scales[(int64_t)p0 * (I >> 7) + (cs[sI] >> 3)];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) {
      for (uint64_t m = pm[k]; m; m &= m - 1) {
        const int p = kWave * k + __builtin_ctzll(m);
        float acc[RPW2];
#pragma unroll
        for (int r = 0; r < RPW2; ++r) acc[r] = 0.0f;
        if (A8 || p == p0) {
#pragma unroll
          for (int sI = 0; sI < NS2; ++sI)
#pragma unroll
            for (int r = 0; r < RPW2; ++r) {
              float sw = scale_value<FMT>(sc[r][sI]);
              if constexpr (A8 || AW) sw *= asc[sI];
              const float n = __builtin_fmaf(chunk_dot_f32<FMT>(w[r][sI], ar[sI]), sw, acc[r]);
              acc[r] = cv[sI] ? n : acc[r];
            }
        } else {
          // further tokens of the expert: activations chunk by chunk from L2
          const float* as = a.a_buf + (int64_t)p * I;
#pragma unroll
          for (int sI = 0; sI < NS2; ++sI) {
            float at[V];
            load_a_chunk(as, sI, at);
            float st = 1.0f;
            if constexpr (AW) st = a.a_scales[(int64_t)p * (I >> 7) + (cs[sI] >> 3)];
#pragma unroll
            for (int r = 0; r < RPW2; ++r) {
              float sw = scale_value<FMT>(sc[r][sI]);
              if constexpr (AW) sw *= st;
              const float n = __builtin_fmaf(chunk_dot_f32<FMT>(w[r][sI], at), sw, acc[r]);
              acc[r] = cv[sI] ? n : acc[r];
            }
          }
        }
#pragma unroll
        for (int r = 0; r < RPW2; ++r) acc[r] = wave_sum_to_last(acc[r]);
        if (lane == kWave - 1) {
          float* dst = a.o_buf + (int64_t)p * H + h0;
#pragma unroll
          for (int r = 0; r < RPW2; ++r) dst[r] = acc[r];
        }
      }
    }
  }
}

// down projection over flattened rows: a unit is R consecutive rows of W2_e, which are one
// contiguous block of R * C2G 8-byte granules, and lane l takes granules l + 64s (s < NSU = R *
// C2G / 64).  Every lane is busy whatever the row length (short rows of tensor-parallel shards
// included) and every load instruction reads 512 contiguous bytes.  Granule l + 64s sits in
// column (l + 64s) mod C2G, which repeats with period D = C2G / gcd(64, C2G) in s, so each lane
// needs only D granules of a; its row is (l + 64s) / C2G, within a few rows of 64s / C2G.
// values per granule of GB bytes
template <int FMT, int GB>
struct Gran {
  static constexpr int kVals = FMT == WFMT_FP8_B128 ? GB : 2 * GB;
};

constexpr int cgcd(int x, int y) { return y == 0 ? x : cgcd(y, x % y); }

// Partial dot product of one 8-byte granule with fp32 activations.
template <int FMT>
__device__ __forceinline__ float granule_dot_f32(uint2 wq, const float* av) {
  opaque(wq);
  const uint32_t ww[2] = {wq.x, wq.y};
  float acc = 0.0f;
  if constexpr (FMT == WFMT_FP8_B128) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x2 lo = fp8x2_to_f32<false>(ww[j]), hi = fp8x2_to_f32<true>(ww[j]);
      acc = __builtin_fmaf(lo.x, av[4 * j], acc);
      acc = __builtin_fmaf(lo.y, av[4 * j + 1], acc);
      acc = __builtin_fmaf(hi.x, av[4 * j + 2], acc);
      acc = __builtin_fmaf(hi.y, av[4 * j + 3], acc);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x2 p0 = fp4x2_to_f32<0>(ww[j]), p1 = fp4x2_to_f32<1>(ww[j]);
      const f32x2 p2 = fp4x2_to_f32<2>(ww[j]), p3 = fp4x2_to_f32<3>(ww[j]);
      acc = __builtin_fmaf(p0.x, av[8 * j], acc);
      acc = __builtin_fmaf(p0.y, av[8 * j + 1], acc);
      acc = __builtin_fmaf(p1.x, av[8 * j + 2], acc);
      acc = __builtin_fmaf(p1.y, av[8 * j + 3], acc);
      acc = __builtin_fmaf(p2.x, av[8 * j + 4], acc);
      acc = __builtin_fmaf(p2.y, av[8 * j + 5], acc);
      acc = __builtin_fmaf(p3.x, av[8 * j + 6], acc);
      acc = __builtin_fmaf(p3.y, av[8 * j + 7], acc);
    }
  }
  return acc;
}

// A8 (W8A8): needs C2G % 64 == 0 and 8-value granules, so that column j of lane l is
// l + 64 j and the 16 granules of one 128-value block of a sit in 16 consecutive lanes.
template <int FMT, int C2G, int NSU, int GB, bool A8>
__global__ __launch_bounds__(kFfnThreads) void down_flat_kernel(FfnArgs a) {
  constexpr int GV = Gran<FMT, GB>::kVals;
  constexpr int D = C2G / cgcd(kWave, C2G);
  constexpr int R = kWave * NSU / C2G;
  static_assert((kWave * NSU) % C2G == 0, "a unit must be whole rows");
  static_assert(FMT != WFMT_FP8_B128 || 128 % R == 0, "a unit must sit in one scale block");
  static_assert(!A8 || (FMT == WFMT_FP8_B128 && C2G % kWave == 0 && GV == 8),
                "W8A8 needs 16 lanes per activation block");
  __shared__ QueueLds QL;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int H = a.H, I = a.I;
  const int gw = blockIdx.x * kFfnWaves + wave;
  const int NW = gridDim.x * kFfnWaves;
  constexpr int64_t rb2 = (int64_t)C2G * GB;
  const int upe = H / R;
  int v0, v1;
  if (a.M == 1) {
    const int U = Q.n_active * upe;
    v0 = (int)((int64_t)U * gw / NW);
    v1 = (int)((int64_t)U * (gw + 1) / NW);
  } else {
    WaveBalance B;
    wave_balance_build(B, Q, QL.cnt[wave], upe, kUnitCost, kPairCost);
    v0 = wave_balance_unit(B, (int64_t)B.total * gw / NW);
    v1 = wave_balance_unit(B, (int64_t)B.total * (gw + 1) / NW);
  }
  int acol[D];  // the columns (granule index within a row) this lane ever touches
#pragma unroll
  for (int j = 0; j < D; ++j) acol[j] = (lane + kWave * j) % C2G;
  auto load_a = [&](const float* as, int j, float (&dst)[GV]) {
#pragma unroll
    for (int k4 = 0; k4 < GV / 4; ++k4) {
      const float4 f = reinterpret_cast<const float4*>(as + (int64_t)acol[j] * GV)[k4];
      dst[4 * k4] = f.x; dst[4 * k4 + 1] = f.y; dst[4 * k4 + 2] = f.z; dst[4 * k4 + 3] = f.w;
    }
  };
  float ar[D][GV];  // first token of the current expert
  float asc[D];     // A8 (one token): their block scales; they serve every pair of the expert
  float one[D];     // unit activation scales of the other pairs without A8
#pragma unroll
  for (int j = 0; j < D; ++j) one[j] = 1.0f;
  uint64_t pm[kPairRegs] = {};
  int cur_q = -1, e = 0, p0 = 0;
  for (int v = v0; v < v1; ++v) {
    const int q = v / upe, h0 = (v % upe) * R;
    const bool fresh = q != cur_q;
    if (fresh) e = wave_queue_expert(Q, q);
    // A8: the new expert's a is loaded before the weights, so that quantizing it waits for
    // those loads only (loads complete in issue order) and overlaps the weight stream
    auto load_first_a = [&]() {
      cur_q = q;
      wave_queue_pairs(Q, q, pm);
      p0 = first_pair(pm);
      const float* as = a.a_buf + (int64_t)p0 * I;
#pragma unroll
      for (int j = 0; j < D; ++j) load_a(as, j, ar[j]);
    };
    if constexpr (A8) {
      if (fresh) load_first_a();
    }
    const uint8_t* base = a.w2 + ((int64_t)e * H + h0) * rb2;
    const void* Ws = scale_ptr<FMT>(a.w2s, (int64_t)e * scale_elems<FMT>(H, I));
    typename std::conditional<GB == 8, uint2, uint4>::type w[NSU];
    // FP8: the unit's R rows lie in one 128-row scale block (R divides 128, units start at
    // multiples of R), so a lane needs only the D scales of its D columns; MXFP4: one per granule
    constexpr int NSC = FMT == WFMT_FP8_B128 ? D : NSU;
    uint32_t sc[NSC];
#pragma unroll
    for (int s = 0; s < NSU; ++s) {
      const int g = lane + kWave * s;
      if constexpr (GB == 8) w[s] = load_stream8(base + (int64_t)g * GB);
      else w[s] = load_stream16(base + (int64_t)g * GB);
    }
    if constexpr (FMT == WFMT_FP8_B128) {
#pragma unroll
      for (int j = 0; j < D; ++j)
        sc[j] = reinterpret_cast<const uint32_t*>(Ws)[(h0 >> 7) * fp8_blocks(I) +
                                                       ((acol[j] * GV) >> 7)];
    } else {
#pragma unroll
      for (int s = 0; s < NSU; ++s) {
        const int row = h0 + (lane + kWave * s) / C2G, col = acol[s % D];
        sc[s] = reinterpret_cast<const uint8_t*>(Ws)[(int64_t)row * (I >> 5) + ((col * GV) >> 5)];
      }
    }
    if (fresh) {
      if constexpr (A8) {
#pragma unroll
        for (int j = 0; j < D; ++j) asc[j] = act_quant_f32<16>(ar[j]);
      } else {
        load_first_a();
      }
    }
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) {
      for (uint64_t m = pm[k]; m; m &= m - 1) {
        const int p = kWave * k + __builtin_ctzll(m);
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
        auto accumulate = [&](const float (&av)[D][GV], const float (&avs)[D]) {
#pragma unroll
          for (int s = 0; s < NSU; ++s) {
            // this granule's row: r0 + ro, ro in [0, kSpan) (one wave spans kSpan rows at most)
            constexpr int kSpan = (kWave + C2G - 1) / C2G + 1;
            const int r0 = kWave * s / C2G;
            const int ro = (lane + kWave * s) / C2G - r0;
            float dot;
            if constexpr (GB == 8) dot = granule_dot_f32<FMT>(w[s], av[s % D]);
            else dot = chunk_dot_f32<FMT>(w[s], av[s % D]);
            float sw = scale_value<FMT>(sc[FMT == WFMT_FP8_B128 ? s % D : s]);
            if constexpr (A8) sw *= avs[s % D];
            const float d = dot * sw;
            if ((kWave * s) % C2G + kWave <= C2G || r0 + 1 >= R) {
              acc[r0] += d;
            } else {
#pragma unroll
              for (int k2 = 0; k2 < kSpan; ++k2)
                if (r0 + k2 < R) acc[r0 + k2] += (ro == k2) ? d : 0.0f;
            }
          }
        };
        if (A8 || p == p0) {
          accumulate(ar, asc);
        } else {  // further tokens of the expert: their granules of a from L2
          const float* as = a.a_buf + (int64_t)p * I;
          float at[D][GV];
#pragma unroll
          for (int j = 0; j < D; ++j) load_a(as, j, at[j]);
          accumulate(at, one);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum_to_last(acc[r]);
        if (lane == kWave - 1) {
          float* dst = a.o_buf + (int64_t)p * H + h0;
#pragma unroll
          for (int r = 0; r < R; ++r) dst[r] = acc[r];
        }
      }
    }
  }
}

// W8A8 with several tokens: the activations are quantized by passes of their own, one thread
// per 8 values and 16 lanes per 128-value block (blocks never straddle a row: H, I % 128 == 0).
// With one token the gate/up and down kernels quantize inside; with several, every pair of a
// unit would repeat the block maxima, so the pass runs once.  x [M][H] -> xq, x_scales.
__global__ __launch_bounds__(256) void act_quant_x_kernel(FfnArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int n8 = a.M * a.H / 8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (c < n8) v = reinterpret_cast<const uint4*>(a.x)[c];
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const float s = act_quant_bf16<16>(w);  // every lane takes part in the group maximum
  if (c < n8) {
    reinterpret_cast<uint4*>(a.xq)[c] = make_uint4(w[0], w[1], w[2], w[3]);
    if ((c & 15) == 0) a.x_scales[c >> 4] = s;
  }
}

// a_buf [M*S][I] -> aq, a_scales [M*S][I/128] (rows of pairs that no valid id names hold
// whatever the buffer held and are never read).  a_buf itself is kept, so a repeated down stage
// on the same gate/up output sees the same input.
__global__ __launch_bounds__(256) void act_quant_a_kernel(FfnArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int n8 = a.M * a.S * a.I / 8;
  float v[8];
  float4 f0 = make_float4(0.f, 0.f, 0.f, 0.f), f1 = f0;
  if (c < n8) {
    f0 = reinterpret_cast<const float4*>(a.a_buf)[2 * c];
    f1 = reinterpret_cast<const float4*>(a.a_buf)[2 * c + 1];
  }
  v[0] = f0.x; v[1] = f0.y; v[2] = f0.z; v[3] = f0.w;
  v[4] = f1.x; v[5] = f1.y; v[6] = f1.z; v[7] = f1.w;
  const float s = act_quant_f32<16>(v);
  if (c < n8) {
    reinterpret_cast<float4*>(a.aq)[2 * c] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(a.aq)[2 * c + 1] = make_float4(v[4], v[5], v[6], v[7]);
    if ((c & 15) == 0) a.a_scales[c >> 4] = s;
  }
}

// y[t][h] = sum over slots j (in order) of w[t][j] * o[t][j][h]; invalid ids contribute nothing.
// RES: y is the residual stream h, updated in place to bf16(h + y).
template <bool RES>
__global__ __launch_bounds__(256) void combine_kernel(FfnArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.M * a.H) return;
  const int t = idx / a.H, h = idx % a.H;
  const uint16_t h_in = RES ? a.y[idx] : 0;
  // all loads first (no branch between them), then the slot-ordered sum
  int e[kMaxSlots];
  float wv[kMaxSlots], ov[kMaxSlots];
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    const int p = t * a.S + (j < a.S ? j : 0);
    e[j] = a.ids[p];
    wv[j] = a.topk_w[p];
    ov[j] = a.o_buf[(int64_t)p * a.H + h];
  }
  float y = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    const bool ok = j < a.S && e[j] >= 0 && e[j] < a.n_experts;
    const float n = __builtin_fmaf(wv[j], ov[j], y);
    y = ok ? n : y;
  }
  if (RES)
    a.y[idx] = f64_to_bf16(bf16_to_f64(h_in) + (double)y);  // h + y, rounded once
  else
    a.y[idx] = f32_to_bf16(y);
}

template <int FMT, int NS, bool A8, bool AW = false>
hipError_t launch_gateup_t(const FfnArgs& a, hipStream_t stream) {
  static int grid = 0;
  auto kern = gateup_kernel<FMT, NS, A8, AW>;
  hipError_t err = resident_grid(kern, &grid);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kFfnThreads), 0, stream, a);
  return hipGetLastError();
}

template <int FMT, int NS2, int RPW2, bool DYN, int TPB, bool A8, bool AW = false>
hipError_t launch_down_kernel(const FfnArgs& a, hipStream_t stream) {
  static int grid = 0;
  auto kern = down_kernel<FMT, NS2, RPW2, DYN, TPB, A8, AW>;
  hipError_t err = resident_grid(kern, &grid, TPB);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(TPB), 0, stream, a);
  return hipGetLastError();
}

// One token: the per-wave split; several tokens: one workgroup per CU, with three waves per
// SIMD for the one-chunk MXFP4 rows (intermediate 2048), two otherwise.  The two MXFP4 row
// lengths whose workgroup-per-CU form would spill (NS2 = 2, 4) keep the per-wave split.
template <int FMT, int NS2, int RPW2, bool A8>
hipError_t launch_down_t(const FfnArgs& a, hipStream_t stream) {
  constexpr bool kCu = !(FMT == WFMT_MXFP4 && (NS2 == 2 || NS2 == 4));
  constexpr int TPB = (FMT == WFMT_MXFP4 && NS2 == 1) ? kCuThreadsWide : kCuThreads;
  if constexpr (A8) {  // W8A8: several tokens read the quantized a from the workspace
    if (a.M > 1) return launch_down_kernel<FMT, NS2, RPW2, true, TPB, false, true>(a, stream);
    return launch_down_kernel<FMT, NS2, RPW2, false, kFfnThreads, true>(a, stream);
  } else {
    if constexpr (kCu) {
      if (a.M > 1) return launch_down_kernel<FMT, NS2, RPW2, true, TPB, false>(a, stream);
    }
    return launch_down_kernel<FMT, NS2, RPW2, false, kFfnThreads, false>(a, stream);
  }
}

template <int FMT, int NS, bool AW = false>
hipError_t launch_gateup_cu_t(const FfnArgs& a, hipStream_t stream) {
  // without spilling, one unit per step fits three waves per SIMD up to NS = 5 (FP8) / 3 (MXFP4)
  constexpr bool kOne = NS <= (FMT == WFMT_FP8_B128 ? 5 : 3);
  constexpr int UPG = kOne ? 1 : 2;
  constexpr int TPB = kOne ? kCuThreadsWide : kCuThreads;
  static int grid = 0;
  auto kern = gateup_cu_kernel<FMT, NS, UPG, TPB, AW>;
  hipError_t err = resident_grid(kern, &grid, TPB);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(TPB), 0, stream, a);
  return hipGetLastError();
}

// One token: the per-wave split (measured faster at M = 1 on both formats; the workgroup-per-CU
// form adds a barrier and an LDS round trip to every step and gained nothing there).  Several
// tokens: one workgroup per CU with dynamic units (1T MXFP4, M = 16: 347 -> 320-326 us; GLM
// MXFP4, M = 4: 61 -> 55 us).
// Chunk counts past NS = 6 (FP8) / 4 (MXFP4) would spill in the workgroup-per-CU form and keep
// the per-wave split.  W8A8 with several tokens reads the quantized x from the workspace, in the
// workgroup-per-CU form up to NS = 6 and the per-wave form past it.
template <int FMT, int NS, bool A8>
hipError_t launch_gateup_ns(const FfnArgs& a, hipStream_t stream) {
  if constexpr (A8) {
    if (a.M != 1) {
      if constexpr (NS <= 6) return launch_gateup_cu_t<FMT, NS, true>(a, stream);
      else return launch_gateup_t<FMT, NS, false, true>(a, stream);
    }
  } else if constexpr (NS <= (FMT == WFMT_FP8_B128 ? 6 : 4)) {
    if (a.M > 1) return launch_gateup_cu_t<FMT, NS>(a, stream);
  }
  return launch_gateup_t<FMT, NS, A8>(a, stream);
}

template <int FMT, bool A8>
hipError_t launch_gateup(const FfnArgs& a, int ns, hipStream_t stream) {
  switch (ns) {
    case 1: return launch_gateup_ns<FMT, 1, A8>(a, stream);
    case 2: return launch_gateup_ns<FMT, 2, A8>(a, stream);
    case 3: return launch_gateup_ns<FMT, 3, A8>(a, stream);
    case 4: return launch_gateup_ns<FMT, 4, A8>(a, stream);
    case 5: return launch_gateup_ns<FMT, 5, A8>(a, stream);
    case 6: return launch_gateup_ns<FMT, 6, A8>(a, stream);
    case 7: return launch_gateup_ns<FMT, 7, A8>(a, stream);
    case 8: return launch_gateup_ns<FMT, 8, A8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, bool A8>
hipError_t launch_down(const FfnArgs& a, int ns2, hipStream_t stream) {
  switch (ns2) {
    case 1: return launch_down_t<FMT, 1, 8, A8>(a, stream);
    case 2: return launch_down_t<FMT, 2, 8, A8>(a, stream);
    case 3: return launch_down_t<FMT, 3, 2, A8>(a, stream);
    case 4: return launch_down_t<FMT, 4, 2, A8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int ffn_chunks_per_lane(int wfmt, int K) {
  const int vals = (wfmt == WFMT_MXFP4) ? 32 : 16;
  return (K / vals + kWave - 1) / kWave;
}

hipError_t launch_gate_up(const FfnArgs& a, int wfmt, hipStream_t stream) {
  const int ns = ffn_chunks_per_lane(wfmt, a.H);
  switch (wfmt) {
    case WFMT_FP8_B128: return launch_gateup<WFMT_FP8_B128, false>(a, ns, stream);
    case WFMT_FP8_B128_A8:
      if (a.M > 1) {  // several tokens: quantize x once into the workspace first
        const int n8 = a.M * a.H / 8;
        hipLaunchKernelGGL(act_quant_x_kernel, dim3((n8 + 255) / 256), dim3(256), 0, stream, a);
      }
      return launch_gateup<WFMT_FP8_B128, true>(a, ns, stream);
    default: return launch_gateup<WFMT_MXFP4, false>(a, ns, stream);
  }
}

template <int FMT, int C2G, int NSU, int GB, bool A8>
hipError_t launch_down_flat_t(const FfnArgs& a, hipStream_t stream) {
  static int grid = 0;
  auto kern = down_flat_kernel<FMT, C2G, NSU, GB, A8>;
  hipError_t err = resident_grid(kern, &grid);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kFfnThreads), 0, stream, a);
  return hipGetLastError();
}

// Flattened-row down projection, one token only, for the row lengths it is instantiated for
// (rows per unit must divide hidden); returns hipErrorNotSupported otherwise.  With several
// tokens the row-chunk kernel with a workgroup per CU measured faster (GLM MXFP4 M = 4,
// down + combine 42.9 -> 39.2 us).
static hipError_t launch_down_flat(const FfnArgs& a, int wfmt, hipStream_t stream) {
  if (a.M > 1) return hipErrorNotSupported;
  if (wfmt == WFMT_FP8_B128) {
    if (a.I == 1536 && a.H % 8 == 0)
      return launch_down_flat_t<WFMT_FP8_B128, 192, 24, 8, false>(a, stream);
    if (a.I == 192 && a.H % 16 == 0)
      return launch_down_flat_t<WFMT_FP8_B128, 24, 6, 8, false>(a, stream);
  } else if (wfmt == WFMT_FP8_B128_A8) {
    if (a.I == 1536 && a.H % 8 == 0)
      return launch_down_flat_t<WFMT_FP8_B128, 192, 24, 8, true>(a, stream);
  } else {
    if (a.I == 1536 && a.H % 8 == 0)
      return launch_down_flat_t<WFMT_MXFP4, 96, 12, 8, false>(a, stream);
    if (a.I == 192 && a.H % 16 == 0)
      return launch_down_flat_t<WFMT_MXFP4, 12, 3, 8, false>(a, stream);
    if (a.I == 256 && a.H % 16 == 0)
      return launch_down_flat_t<WFMT_MXFP4, 16, 4, 8, false>(a, stream);
  }
  return hipErrorNotSupported;
}

hipError_t launch_down_combine(const FfnArgs& a, int wfmt, hipStream_t stream) {
  hipError_t err = launch_down_flat(a, wfmt, stream);
  if (err == hipErrorNotSupported) {
    const int ns2 = ffn_chunks_per_lane(wfmt, a.I);
    switch (wfmt) {
      case WFMT_FP8_B128: err = launch_down<WFMT_FP8_B128, false>(a, ns2, stream); break;
      case WFMT_FP8_B128_A8:
        if (a.M > 1) {  // several tokens: quantize a once into aq, which the down kernel reads
          const int n8 = a.M * a.S * a.I / 8;
          hipLaunchKernelGGL(act_quant_a_kernel, dim3((n8 + 255) / 256), dim3(256), 0, stream,
                             a);
          FfnArgs q = a;
          q.a_buf = a.aq;
          err = launch_down<WFMT_FP8_B128, true>(q, ns2, stream);
        } else {
          err = launch_down<WFMT_FP8_B128, true>(a, ns2, stream);
        }
        break;
      default: err = launch_down<WFMT_MXFP4, false>(a, ns2, stream); break;
    }
  }
  if (err != hipSuccess) return err;
  const int n = a.M * a.H;
  if (a.residual)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((n + 255) / 256), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((n + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
