// Device bodies of the expert-FFN kernels, shared by the stage kernels (ffn.hip) and the
// one-launch one-token layer (layer_m1.hip): weight-chunk dot products, gate/up + SwiGLU over
// a range of units, and the two down projections over a range of units.
//   molayo1419.me Xiaomi 1T page, section 1: decode reads every active weight from HBM once per
//   step and is bound by bandwidth; section 2: expert FFN weights in MXFP4.
//   d9249.github.io "glm-5-2-b300-kernel-mtp-serving", table under "what it solves" and idea 1:
//   a batch-1 expert GEMM needs many long concurrent memory streams to approach peak bandwidth;
//   idea 2: scale handling must not stall the load pipeline; idea 3: a verify block of M tokens
//   shares one weight stream.
#pragma once
#include <type_traits>

#include "act_quant.h"
#include "ffn_common.h"
#include "route_select.h"

namespace moe {
namespace {

// ---- hand-off of the intermediate results (a, o) between the waves that produce and use them
// PlainIO: producer and consumer are separate launches, ordered by the kernel boundary; a value
// is a plain fp32 element of the buffer.
struct PlainIO {
  static constexpr bool kLaunch = false;
  __device__ void put(float* base, int64_t i, float v) const { base[i] = v; }
  __device__ float4 get4(const float* base, int64_t i, bool&) const {
    return *reinterpret_cast<const float4*>(base + i);
  }
  // waits until value i is there (nothing to wait for after a kernel boundary)
  __device__ void probe(const float*, int64_t) const {}
  // whether the values just loaded are complete (always, after a kernel boundary)
  __device__ bool ready(bool, int) const { return true; }
};

// LaunchIO: producer and consumer are waves of one launch, possibly on different XCDs, whose L2
// caches are not kept coherent with each other.  Value i is the 64-bit word i of the buffer:
// the fp32 bits in the low half, the launch's epoch (a per-call number) in the high half, written
// and read with relaxed device-scope atomics (which the L2 neither keeps dirty nor serves
// stale).  A consumer reloads until every word it needs carries the current epoch, so no
// counter, fence or reset is needed between producer and consumer, and words left by earlier
// calls never pass for current ones.  A wait that does not end within kSpinLimit polls sets
// bit 1 of the status word and gives up (it cannot happen while the whole grid is resident),
// so every wave always exits.
constexpr int kSpinLimit = 1 << 18;

struct LaunchIO {
  static constexpr bool kLaunch = true;
  uint32_t epoch;
  int32_t* status;
  __device__ void put(float* base, int64_t i, float v) const {
    const uint64_t w = ((uint64_t)epoch << 32) | __float_as_uint(v);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(base) + i, w, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ float get1(const float* base, int64_t i, bool& ok) const {
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(base)) + i;
    const uint64_t w = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = ok && (uint32_t)(w >> 32) == epoch;
    return __uint_as_float((uint32_t)w);
  }
  __device__ float4 get4(const float* base, int64_t i, bool& ok) const {
    float4 f;
    f.x = get1(base, i, ok);
    f.y = get1(base, i + 1, ok);
    f.z = get1(base, i + 2, ok);
    f.w = get1(base, i + 3, ok);
    return f;
  }
  // true when every lane's loads carried the epoch (or the wait gave up); else sleep about a
  // microsecond, so that waiting waves load little while the others stream their weights
  __device__ bool ready(bool ok, int it) const {
    if (__ballot(!ok) == 0) return true;
    if (it >= kSpinLimit) {
      if (threadIdx.x % kWave == 0 && status) atomicOr(status, 2);
      return true;
    }
    __builtin_amdgcn_s_sleep(40);
    return false;
  }
  // waits until every lane's value i carries the epoch: one word per lane per poll, before the
  // caller loads (and checks) all it needs
  __device__ void probe(const float* base, int64_t i) const {
    for (int it = 0;; ++it) {
      bool ok = true;
      get1(base, i, ok);
      if (ready(ok, it)) break;
    }
  }
};

// Per-unit hook of the down bodies (the one-launch layer combines the rows whose last unit a
// wave finished); the stage kernels do nothing there.
struct NoReport {
  __device__ void unit_done(int, int) {}
  __device__ void finish() {}
};

// Partial dot product of one 16-byte weight chunk with bf16 activations (kXWords pairs).
// The chunk passes through opaque() so its decode stays inside the caller's per-token loop.
// The work queue of a wave of an NWV-wave workgroup with several tokens: from the routing ids,
// or (logits set) from the workgroup's own selection (select_tokens into sel, LDS [M * S]; the
// grid's first workgroup publishes ids and weights).  Every wave of the workgroup must call it:
// the selection ends at a workgroup barrier.
template <int NWV>
__device__ __forceinline__ void tokens_queue(const FfnArgs& a, WaveQueue& Q, uint32_t* bits,
                                             int* base, int* sel) {
  if (a.logits == nullptr) {
    wave_queue_build(Q, bits, base, a.ids, a.M * a.S, a.n_experts);
    return;
  }
  select_tokens<NWV>(a.logits, a.M, a.E_routed, a.k_routed, a.S - a.k_routed, sel,
                     blockIdx.x == 0, a.ids_out, a.w_out);
  __syncthreads();
  wave_queue_build(Q, bits, base, sel, a.M * a.S, a.n_experts);
}

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
// The range [u0, u1) is the wave's share of the n_active * I units; io stores the values.
template <int FMT, int NS, class IO = PlainIO>
__device__ void gateup_one_token(const FfnArgs& a, const WaveQueue& Q, int u0, int u1,
                                 const IO& io = IO()) {
  constexpr int V = Fmt<FMT>::kVals;
  constexpr int XW = Fmt<FMT>::kXWords;
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I;
  const int C = H / V;
  const int64_t rb = Fmt<FMT>::row_bytes(H);
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
          io.put(a.a_buf, outi, outv);
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
  if (lane < nout) io.put(a.a_buf, outi, outv);
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
// The body over the units [u0, u1) (DYN: the workgroup's range, whose units its waves take from
// `next`); io stores the values.
template <int FMT, int NS, int UPG, bool DYN, bool A8, bool AW, class IO = PlainIO>
__device__ __forceinline__ void gateup_range(const FfnArgs& a, const WaveQueue& Q, int* next,
                                             int u0, int u1, ActLds* xl,
                                             const ActX<kFfnThreads, (NS + 1) / 2>* xv,
                                             const IO& io = IO()) {
  static_assert(UPG == 1 || UPG == 2, "one or two units per iteration");
  static_assert(!A8 || FMT == WFMT_FP8_B128, "W8A8 takes FP8 weights");
  constexpr int V = Fmt<FMT>::kVals;
  constexpr int XW = Fmt<FMT>::kXWords;
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I, S = a.S;
  const int C = H / V;
  const int64_t rb = Fmt<FMT>::row_bytes(H);
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
            if (lane == kWave - 1) io.put(a.a_buf, (int64_t)p * I + i + d, silu_mul(g, up));
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

// ---- several tokens with every token's activations in LDS
// x [M][H] bf16 in LDS, each chunk's 16-byte pieces rotated by the chunk's index over the array
// (piece k of chunk c at slot (k + c) mod P, P pieces per chunk), so that the lanes of a wave,
// reading piece k of consecutive chunks, fall on different banks.  Capacity: 7 tokens of hidden
// 7168 (from 8 tokens on, the matrix-core launch takes the supported shapes).
constexpr int kXlBytes = 7 * 7168 * 2;

template <int FMT, int TPB>
__device__ __forceinline__ void xl_stage(const FfnArgs& a, uint4* xl) {
  constexpr int P = Fmt<FMT>::kXWords / 4;
  const int n16 = a.M * a.H / 8;
  const uint4* src = reinterpret_cast<const uint4*>(a.x);
  for (int i0 = threadIdx.x; i0 < n16; i0 += 4 * TPB) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * TPB;
      v[j] = src[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * TPB, c = i / P;
      if (i < n16) xl[c * P + (i + c) % P] = v[j];
    }
  }
}

// gate/up + SwiGLU with several tokens, every pair's activations from the LDS copy (xl_stage):
// the registers hold no activations, so more waves fit per SIMD.  The workgroup's waves take UPG
// units at a time from the LDS counter `next` until u1, as gateup_range with DYN; per unit and
// pair the arithmetic, and its order, is gateup_range's, so the values are the same bits.
template <int FMT, int NS, int UPG>
__device__ __forceinline__ void gateup_xl_range(const FfnArgs& a, const WaveQueue& Q, int* next,
                                                int u1, const uint4* xl) {
  static_assert(UPG == 1 || UPG == 2, "one or two units per iteration");
  constexpr int V = Fmt<FMT>::kVals;
  constexpr int XW = Fmt<FMT>::kXWords;
  constexpr int P = XW / 4;
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I, S = a.S;
  const int C = H / V;
  const int64_t rb = Fmt<FMT>::row_bytes(H);
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(next, UPG);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int cs[NS];
  bool cv[NS];
#pragma unroll
  for (int sI = 0; sI < NS; ++sI) {
    const int c = lane + kWave * sI;
    cv[sI] = c < C;
    cs[sI] = cv[sI] ? c : C - 1;
  }
  // chunk sI of this lane of token t's activations
  auto load_x = [&](int t, int sI, uint32_t (&dst)[XW]) {
    const int c = t * C + cs[sI];
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const uint4 v = xl[c * P + (k + c) % P];
      dst[4 * k] = v.x; dst[4 * k + 1] = v.y; dst[4 * k + 2] = v.z; dst[4 * k + 3] = v.w;
    }
  };
  uint64_t pm[kPairRegs] = {};
  int cur_q = -1, e = 0;
  for (int u = grab(); u < u1; u = grab()) {
    const int q = u / I, i = u % I;
    if (q != cur_q) e = wave_queue_expert(Q, q);
    const int nu = (UPG == 2 && u + 1 < u1 && i + 1 < I) ? 2 : 1;  // units this iteration
    const uint8_t* W = a.w13 + (int64_t)e * 2 * I * rb;
    const void* Ws = scale_ptr<FMT>(a.w13s, (int64_t)e * scale_elems<FMT>(2 * I, H));
    uint4 w[2][2][NS];  // [unit][gate, up][chunk]
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
    if (q != cur_q) {
      cur_q = q;
      wave_queue_pairs(Q, q, pm);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (d < nu) {
#pragma unroll
        for (int k = 0; k < kPairRegs; ++k) {
          for (uint64_t m = pm[k]; m; m &= m - 1) {
            const int p = kWave * k + __builtin_ctzll(m);
            float g = 0.0f, up = 0.0f;
#pragma unroll
            for (int sI = 0; sI < NS; ++sI) {
              uint32_t xt[XW];
              load_x(p / S, sI, xt);
              const float ng = __builtin_fmaf(chunk_dot_bf16<FMT>(w[d][0][sI], xt),
                                              scale_value<FMT>(sc[d][0][sI]), g);
              const float nu2 = __builtin_fmaf(chunk_dot_bf16<FMT>(w[d][1][sI], xt),
                                               scale_value<FMT>(sc[d][1][sI]), up);
              g = cv[sI] ? ng : g;
              up = cv[sI] ? nu2 : up;
            }
            g = wave_sum_to_last(g);
            up = wave_sum_to_last(up);
            if (lane == kWave - 1) a.a_buf[(int64_t)p * I + i + d] = silu_mul(g, up);
          }
        }
      }
    }
  }
}

// Part `part` of `nparts` of the gate/up units: one token, a plain split; several tokens, the
// cost-weighted split (a unit costs one pass per pair).
template <int FMT, int NS, int UPG, bool DYN, bool A8, bool AW = false>
__device__ __forceinline__ void gateup_tokens(const FfnArgs& a, const WaveQueue& Q, int* cnt,
                                              int* next, int part, int nparts,
                                              ActLds* xl = nullptr,
                                              const ActX<kFfnThreads, (NS + 1) / 2>* xv = nullptr) {
  // with UPG = 2 and DYN the part boundaries sit at even units
  constexpr int kAlign = (DYN && UPG == 2) ? ~1 : ~0;
  int u0, u1;
  if (a.M == 1) {
    const int U = Q.n_active * a.I;
    u0 = (int)((int64_t)U * part / nparts) & kAlign;
    u1 = (int)((int64_t)U * (part + 1) / nparts) & kAlign;
  } else {
    WaveBalance B;
    wave_balance_build(B, Q, cnt, a.I, kUnitCost, kPairCost);
    u0 = wave_balance_unit(B, (int64_t)B.total * part / nparts) & kAlign;
    u1 = wave_balance_unit(B, (int64_t)B.total * (part + 1) / nparts) & kAlign;
  }
  gateup_range<FMT, NS, UPG, DYN, A8, AW>(a, Q, next, u0, u1, xl, xv);
}


// down projection: each iteration takes RPW2 consecutive rows of one expert, over the units
// [v0, v1) (DYN: the workgroup's range, whose units its waves take from `next` one at a time).
// AW: W8A8 with several tokens: a_buf already holds the quantized values and a_scales their
// block scales (a pass of their own).  io loads a and stores o; rep sees every finished unit
// (the one-launch layer, DYN = false).
template <int FMT, int NS2, int RPW2, bool DYN, bool A8, bool AW, class IO = PlainIO,
          class Rep = NoReport>
__device__ __forceinline__ void down_rows_range(const FfnArgs& a, const WaveQueue& Q, int* next,
                                                int v0, int v1, Rep& rep, const IO& io = IO()) {
  static_assert(!A8 || FMT == WFMT_FP8_B128, "W8A8 takes FP8 weights");
  constexpr int V = Fmt<FMT>::kVals;
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I;
  const int C2 = I / V;
  const int64_t rb2 = Fmt<FMT>::row_bytes(I);
  const int units_per_expert = H / RPW2;
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(next, 1);
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
  // chunk sI of this lane of pair p's a (reloaded until complete, see LaunchIO)
  auto load_a_chunk = [&](int p, int sI, float (&dst)[V]) {
    io.probe(a.a_buf, (int64_t)p * I + (int64_t)cs[sI] * V + V - 1);
    for (int it = 0;; ++it) {
      bool ok = true;
#pragma unroll
      for (int k4 = 0; k4 < V / 4; ++k4) {
        const float4 f = io.get4(a.a_buf, (int64_t)p * I + (int64_t)cs[sI] * V + 4 * k4, ok);
        dst[4 * k4] = f.x; dst[4 * k4 + 1] = f.y; dst[4 * k4 + 2] = f.z; dst[4 * k4 + 3] = f.w;
      }
      if (io.ready(ok, it)) break;
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
    // A8: the new expert's a is loaded before the weights (see down_flat_range); otherwise after
    // them, so that a wait for the expert's gate/up values (the one-launch layer) overlaps the
    // weight loads
    auto load_first_a = [&]() {
      cur_q = q;
      wave_queue_pairs(Q, q, pm);
      p0 = first_pair(pm);
      io.probe(a.a_buf, (int64_t)p0 * I + (int64_t)cs[NS2 - 1] * V + V - 1);
      for (int it = 0;; ++it) {
        bool ok = true;
#pragma unroll
        for (int sI = 0; sI < NS2; ++sI)
#pragma unroll
          for (int k4 = 0; k4 < V / 4; ++k4) {
            const float4 f =
                io.get4(a.a_buf, (int64_t)p0 * I + (int64_t)cs[sI] * V + 4 * k4, ok);
            ar[sI][4 * k4] = f.x; ar[sI][4 * k4 + 1] = f.y;
            ar[sI][4 * k4 + 2] = f.z; ar[sI][4 * k4 + 3] = f.w;
          }
        if (io.ready(ok, it)) break;
      }
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
#pragma unroll
          for (int sI = 0; sI < NS2; ++sI) {
            float at[V];
            load_a_chunk(p, sI, at);
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
#pragma unroll
          for (int r = 0; r < RPW2; ++r) io.put(a.o_buf, (int64_t)p * H + h0 + r, acc[r]);
        }
      }
    }
    rep.unit_done(q, h0);
  }
  rep.finish();
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

// The flattened-row body over the units [v0, v1) of one wave.  A8 (W8A8): needs C2G % 64 == 0
// and 8-value granules, so that column j of lane l is l + 64 j and the 16 granules of one
// 128-value block of a sit in 16 consecutive lanes.  io loads a and stores o; rep sees every
// finished unit (the one-launch layer).
template <int FMT, int C2G, int NSU, int GB, bool A8, class IO = PlainIO, class Rep = NoReport>
__device__ __forceinline__ void down_flat_range(const FfnArgs& a, const WaveQueue& Q, int v0,
                                                int v1, Rep& rep, const IO& io = IO()) {
  constexpr int GV = Gran<FMT, GB>::kVals;
  constexpr int D = C2G / cgcd(kWave, C2G);
  constexpr int R = kWave * NSU / C2G;
  static_assert((kWave * NSU) % C2G == 0, "a unit must be whole rows");
  static_assert(FMT != WFMT_FP8_B128 || 128 % R == 0, "a unit must sit in one scale block");
  static_assert(!A8 || (FMT == WFMT_FP8_B128 && C2G % kWave == 0 && GV == 8),
                "W8A8 needs 16 lanes per activation block");
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I;
  constexpr int64_t rb2 = (int64_t)C2G * GB;
  const int upe = H / R;
  int acol[D];  // the columns (granule index within a row) this lane ever touches
#pragma unroll
  for (int j = 0; j < D; ++j) acol[j] = (lane + kWave * j) % C2G;
  // this lane's D granule columns of pair p's a (reloaded until complete, see LaunchIO)
  auto load_a_all = [&](int p, float (&dst)[D][GV]) {
    io.probe(a.a_buf, (int64_t)p * I + (int64_t)acol[D - 1] * GV + GV - 1);
    for (int it = 0;; ++it) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < D; ++j)
#pragma unroll
        for (int k4 = 0; k4 < GV / 4; ++k4) {
          const float4 f = io.get4(a.a_buf, (int64_t)p * I + (int64_t)acol[j] * GV + 4 * k4, ok);
          dst[j][4 * k4] = f.x; dst[j][4 * k4 + 1] = f.y;
          dst[j][4 * k4 + 2] = f.z; dst[j][4 * k4 + 3] = f.w;
        }
      if (io.ready(ok, it)) break;
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
      load_a_all(p0, ar);
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
          float at[D][GV];
          load_a_all(p, at);
          accumulate(at, one);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum_to_last(acc[r]);
        if (lane == kWave - 1) {
#pragma unroll
          for (int r = 0; r < R; ++r) io.put(a.o_buf, (int64_t)p * H + h0 + r, acc[r]);
        }
      }
    }
    rep.unit_done(q, h0);
  }
  rep.finish();
}

// The flattened-row body with several tokens: [v0, v1) is the workgroup's range, whose units its
// waves take one at a time from the LDS counter `next`.  The first pair's a of the current
// expert sits in this wave's LDS row `al` (C2G * GV = I floats) rather than in registers, which
// lets the kernel run three waves per SIMD.  (Measured on the GLM MXFP4 layer at 4 tokens: 38.5
// us with a in registers at two waves per SIMD, 33.5 us this way; a second unit in flight per
// wave, software-pipelined, was slower at either occupancy.)  Per unit and pair the arithmetic,
// and its order, is that of down_flat_range.
template <int FMT, int C2G, int NSU, int GB>
__device__ __forceinline__ void down_flat_dyn(const FfnArgs& a, const WaveQueue& Q, int v1,
                                              int* next, float* al) {
  constexpr int GV = Gran<FMT, GB>::kVals;
  constexpr int D = C2G / cgcd(kWave, C2G);
  constexpr int R = kWave * NSU / C2G;
  static_assert(FMT == WFMT_MXFP4 && GB == 8 && C2G % 2 == 0,
                "MXFP4 rows of 8-byte granules: two granules per scale byte");
  static_assert((kWave * NSU) % C2G == 0, "a unit must be whole rows");
  static_assert((C2G * GV) % (4 * kWave) == 0, "a row of a is whole 16-byte pieces per lane");
  struct Unit {
    uint2 w[NSU];
    uint32_t sc[NSU];
  };
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I;
  constexpr int rb2 = C2G * GB;
  const int upe = H / R;
  int acol[D];
#pragma unroll
  for (int j = 0; j < D; ++j) acol[j] = (lane + kWave * j) % C2G;
  // Granule g = lane + 64 s of the unit's contiguous R * C2G granules sits at byte 8 g; its scale
  // byte (row g / C2G, column g % C2G of the unit, two granules per byte, C2G / 2 bytes per row)
  // at byte g / 2 of the unit's contiguous scale bytes.
  auto load_unit = [&](Unit& u, int v) {
    const int q = v / upe, h0 = (v % upe) * R;
    const int e = wave_queue_expert(Q, q);
    const uint8_t* wb = a.w2 + ((int64_t)e * H + h0) * rb2;
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.w2s) +
                        ((int64_t)e * H + h0) * (C2G / 2);
#pragma unroll
    for (int s = 0; s < NSU; ++s) u.w[s] = load_stream8(wb + 8 * lane + 512 * s);
#pragma unroll
    for (int s = 0; s < NSU; ++s) u.sc[s] = sb[(lane >> 1) + 32 * s];
  };
  uint64_t pm[kPairRegs] = {};
  int cur_q = -1, p0 = 0;
  auto run_unit = [&](const Unit& u, int v) {
    const int q = v / upe, h0 = (v % upe) * R;
    if (q != cur_q) {  // a new expert: its first pair's a into this wave's LDS row
      cur_q = q;
      wave_queue_pairs(Q, q, pm);
      p0 = first_pair(pm);
      constexpr int kPer = C2G * GV / (4 * kWave);
      float4 t[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        t[k] = reinterpret_cast<const float4*>(a.a_buf + (int64_t)p0 * I)[lane + kWave * k];
#pragma unroll
      for (int k = 0; k < kPer; ++k) reinterpret_cast<float4*>(al)[lane + kWave * k] = t[k];
    }
    // pair p over this unit with this lane's D granule columns of its a in av
    auto pair_unit = [&](int p, const float (&av)[D][GV]) {
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int s = 0; s < NSU; ++s) {
        constexpr int kSpan = (kWave + C2G - 1) / C2G + 1;
        const int r0 = kWave * s / C2G;
        const int ro = (lane + kWave * s) / C2G - r0;
        float dot;
        if constexpr (GB == 8) dot = granule_dot_f32<FMT>(u.w[s], av[s % D]);
        else dot = chunk_dot_f32<FMT>(u.w[s], av[s % D]);
        const float d = dot * scale_value<FMT>(u.sc[s]);
        if ((kWave * s) % C2G + kWave <= C2G || r0 + 1 >= R) {
          acc[r0] += d;
        } else {
#pragma unroll
          for (int k2 = 0; k2 < kSpan; ++k2)
            if (r0 + k2 < R) acc[r0 + k2] += (ro == k2) ? d : 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = wave_sum_to_last(acc[r]);
      if (lane == kWave - 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) a.o_buf[(int64_t)p * H + h0 + r] = acc[r];
      }
    };
    // the first pair from LDS, as its own block: were it a branch beside the L2 reads of the
    // further pairs, the compiler would merge the two into flat reads, which also wait for the
    // prefetched weights
    {
      typedef float f32x4v __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) const f32x4v lds_f32x4;
      float av[D][GV];
#pragma unroll
      for (int j = 0; j < D; ++j)
#pragma unroll
        for (int k4 = 0; k4 < GV / 4; ++k4) {
          const f32x4v f = *(lds_f32x4*)(al + acol[j] * GV + 4 * k4);
          av[j][4 * k4] = f.x; av[j][4 * k4 + 1] = f.y;
          av[j][4 * k4 + 2] = f.z; av[j][4 * k4 + 3] = f.w;
        }
      pair_unit(p0, av);
    }
    // further tokens of the expert, in pair order: their granules of a from L2
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) {
      for (uint64_t m = pm[k]; m; m &= m - 1) {
        const int p = kWave * k + __builtin_ctzll(m);
        if (p == p0) continue;
        const float* src = a.a_buf + (int64_t)p * I;
        float av[D][GV];
#pragma unroll
        for (int j = 0; j < D; ++j)
#pragma unroll
          for (int k4 = 0; k4 < GV / 4; ++k4) {
            const float4 f = *reinterpret_cast<const float4*>(src + acol[j] * GV + 4 * k4);
            av[j][4 * k4] = f.x; av[j][4 * k4 + 1] = f.y;
            av[j][4 * k4 + 2] = f.z; av[j][4 * k4 + 3] = f.w;
          }
        pair_unit(p, av);
      }
    }
  };
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(next, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  for (int v = grab(); v < v1; v = grab()) {
    Unit u;
    load_unit(u, v);
    run_unit(u, v);
  }
}


}  // namespace
}  // namespace moe
