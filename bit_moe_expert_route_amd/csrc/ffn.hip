// Expert FFN decode as three stream-ordered launches of persistent grids: stream each active
// expert's packed W13 and W2 once, SwiGLU in between, weighted combine in slot order.  (From 8
// tokens on, the gate/up and down launches of ffn_mfma.hip replace the first two.)
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

#include "ffn_body.h"
#include "route_select.h"

namespace moe {
namespace {

// One token with MXFP4 weights takes the pipelined body: half the bytes per row of FP8 make a
// wave's batches short, and batch count (not bytes) set its time (measured: 33.3 -> 30.3 us on
// the 1T-class gate/up).  With FP8 weights the two bodies measured the same.
// AW: W8A8 with several tokens at chunk counts whose workgroup-per-CU form would spill (x and
// its scales quantized into the workspace beforehand).
template <int FMT, int NS, bool AW = false>
__device__ __forceinline__ void gateup_body(const FfnArgs& a, const WaveQueue& Q, int* cnt,
                                            int gw, int NW) {
  if (FMT == WFMT_MXFP4 && a.M == 1) {
    const int U = Q.n_active * a.I;
    gateup_one_token<FMT, NS>(a, Q, (int)((int64_t)U * gw / NW), (int)((int64_t)U * (gw + 1) / NW));
  } else
    gateup_tokens<FMT, NS, 2, false, false, AW>(a, Q, cnt, nullptr, gw, NW);
}

// gate/up of the experts the routing ids in global memory name.
// The work queue of a gate/up wave: from the routing ids, or (one token, logits set) from the
// wave's own selection over the logits, whose result the grid's first wave publishes, or
// (several tokens, logits set) from the workgroup's selection (tokens_queue).  The selection's
// register arrays are sized by the experts per lane (3, 6 or 16).
__device__ __forceinline__ void gateup_queue(const FfnArgs& a, WaveQueue& Q, uint32_t* bits,
                                             int* base, int* sel) {
  if (a.logits == nullptr || a.M > 1) {
    tokens_queue<kFfnWaves>(a, Q, bits, base, sel);
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

// Persistent grids of several workgroups per CU with a static split: the waves of the workgroups
// resident after a CU's first one take a higher issue priority.  Under oldest-first arbitration
// the first workgroup's waves otherwise run ahead and the later ones, with the same work, end
// the kernel 2-5 us later.  Used by the one-token FP8 (bf16 activation) gate/up and down, where
// it measured 0.4-1.4 us faster per launch of the gate/up; the W8A8 and MXFP4 one-token bodies
// measured slower with it.  Workgroups below the CU count are the first on their CUs.
__device__ __forceinline__ void resident_priority(const FfnArgs& a) {
  if ((int)blockIdx.x >= a.cus) __builtin_amdgcn_s_setprio(1);
}

// Loads that only some waves use are issued by all through wave_rsrc, with n = 0 for the waves
// that do not use them (their loads then return zero without touching memory): unconditional
// loads keep the compiler's wait for earlier loads from waiting for these as well, which a load
// under a branch would not.

// One token, FP8 weights, bf16 activations, a shared expert: its units are known before the
// routing, so wave g loads unit g of it (gate and up rows, their scales, the token's
// activations) right behind its routing loads (the logits it selects from, or the ids); those
// bytes stream while the wave selects and builds its queue.  Waves g < I then compute that unit
// (the arithmetic of gateup_range, per chunk and in the same order, so the values are the same
// bits), and every wave its share of the other experts' units, shares balanced so that shared
// plus other units per wave follow the plain split of all units.  The weight loads of waves
// g >= I read nothing (wave_rsrc).  When the queue does not end with the shared expert holding
// one pair (ids given by the caller), the plain split of gateup_tokens.  Requires
// I <= waves <= S * I.
template <int NS>
__device__ __forceinline__ void gateup_shared_first(const FfnArgs& a, uint32_t* bits, int* base,
                                                    int gw, int NW) {
  constexpr int FMT = WFMT_FP8_B128;
  constexpr int XW = Fmt<FMT>::kXWords;
  const int lane = threadIdx.x % kWave;
  const int H = a.H, I = a.I, S = a.S, C = H / Fmt<FMT>::kVals;
  const int64_t rb = Fmt<FMT>::row_bytes(H);
  const int es = a.n_experts - 1;  // the shared expert
  gw = __builtin_amdgcn_readfirstlane(gw);
  const bool mine = gw < I;
  const int i = mine ? gw : 0;
  int cs[NS];
  bool cv[NS];
#pragma unroll
  for (int sI = 0; sI < NS; ++sI) {
    const int c = lane + kWave * sI;
    cv[sI] = c < C;
    cs[sI] = cv[sI] ? c : C - 1;
  }
  uint4 w[2][NS];
  uint32_t sc[2][NS];
  uint32_t xr[NS][XW];
  auto pre = [&]() {
    const uint8_t* W = a.w13 + (int64_t)es * 2 * I * rb;
    const void* Ws = scale_ptr<FMT>(a.w13s, (int64_t)es * scale_elems<FMT>(2 * I, H));
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = r * I + i;
      const __amdgpu_buffer_rsrc_t rs = wave_rsrc(W + (int64_t)row * rb, mine ? (int)rb : 0);
#pragma unroll
      for (int sI = 0; sI < NS; ++sI) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, cs[sI] * 16, 0, kNonTemporal);
        w[r][sI] = make_uint4(q.x, q.y, q.z, q.w);
        sc[r][sI] = scale_raw<FMT>(Ws, H, row, cs[sI]);
      }
    }
    const uint32_t* xs = reinterpret_cast<const uint32_t*>(a.x);
#pragma unroll
    for (int sI = 0; sI < NS; ++sI)
#pragma unroll
      for (int k4 = 0; k4 < XW / 4; ++k4) {
        const uint4 v = reinterpret_cast<const uint4*>(xs + (int64_t)cs[sI] * XW)[k4];
        xr[sI][4 * k4] = v.x; xr[sI][4 * k4 + 1] = v.y;
        xr[sI][4 * k4 + 2] = v.z; xr[sI][4 * k4 + 3] = v.w;
      }
  };
  int v[kPairRegs];
  if (a.logits == nullptr) {
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) {
      const int j = lane + kWave * k;
      v[k] = a.ids[j < S ? j : S - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    pre();
    __builtin_amdgcn_sched_barrier(0);
  } else {
    const int per = (a.E_routed + kWave - 1) / kWave;
    const bool pub = blockIdx.x == 0 && threadIdx.x < kWave;
    int id;
    float wt;
    if (per <= 3)
      wave_select<3, false, decltype(pre)>(a.logits, a.E_routed, a.k_routed, a.has_shared, id,
                                           wt, pub, nullptr, pre);
    else if (per <= 6)
      wave_select<6, false, decltype(pre)>(a.logits, a.E_routed, a.k_routed, a.has_shared, id,
                                           wt, pub, nullptr, pre);
    else
      wave_select<(kMaxExperts + kWave - 2) / kWave, false, decltype(pre)>(
          a.logits, a.E_routed, a.k_routed, a.has_shared, id, wt, pub, nullptr, pre);
    if (pub && lane < S) {
      a.ids_out[lane] = id;
      a.w_out[lane] = wt;
    }
    v[0] = id;
#pragma unroll
    for (int k = 1; k < kPairRegs; ++k) v[k] = -1;
  }
  WaveQueue Q;
  wave_queue_from(Q, bits, base, v, S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int n = Q.n_active, T = n * I, Ur = (n - 1) * I;
  // the shared expert last, with one pair (token 0, slot p), and at least a unit per wave
  bool ok = !Q.invalid && n >= 1 && T >= NW;
  if (ok) ok = wave_queue_expert(Q, n - 1) == es;
  int p = 0;
  if (ok) {
    uint64_t pm[kPairRegs];
    wave_queue_pairs(Q, n - 1, pm);
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) cnt += __popcll(pm[k]);
    ok = cnt == 1;
    p = first_pair(pm);
  }
  if (!ok) {
    gateup_range<FMT, NS, 2, false, false, false>(a, Q, nullptr, (int)((int64_t)T * gw / NW),
                                                  (int)((int64_t)T * (gw + 1) / NW), nullptr,
                                                  nullptr);
    return;
  }
  if (gw < I) {
    float g = 0.0f, up = 0.0f;
#pragma unroll
    for (int sI = 0; sI < NS; ++sI) {
      const float sg = scale_value<FMT>(sc[0][sI]), su = scale_value<FMT>(sc[1][sI]);
      const float ng = __builtin_fmaf(chunk_dot_bf16<FMT>(w[0][sI], xr[sI]), sg, g);
      const float nu2 = __builtin_fmaf(chunk_dot_bf16<FMT>(w[1][sI], xr[sI]), su, up);
      g = cv[sI] ? ng : g;
      up = cv[sI] ? nu2 : up;
    }
    g = wave_sum_to_last(g);
    up = wave_sum_to_last(up);
    if (lane == kWave - 1) a.a_buf[(int64_t)p * I + i] = silu_mul(g, up);
  }
  // wave g's first unit of the others: its start in the plain split less the shared units of
  // the waves before it (non-decreasing in g as T >= NW)
  auto start = [&](int g) {
    const int s = (int)((int64_t)T * g / NW) - (g < I ? g : I);
    return s < 0 ? 0 : (s > Ur ? Ur : s);
  };
  gateup_range<FMT, NS, 2, false, false, false>(a, Q, nullptr, start(gw), start(gw + 1), nullptr,
                                                nullptr);
}

// A8 (one token): the workgroup stages the token's quantized activations in LDS.  AW: several
// W8A8 tokens read from the workspace (per-wave split).
template <int FMT, int NS, bool A8, bool AW = false>
__global__ __launch_bounds__(kFfnThreads) void gateup_kernel(FfnArgs a) {
  static_assert(!(A8 && AW), "one token or several");
  __shared__ QueueLds QL;
  __shared__ int SEL[kMaxPairs];
  __shared__ typename std::conditional<A8, ActLds, char>::type XL;
  // NS chunks of 16 values per lane cover H, so (NS + 1) / 2 pieces of 8 per thread do
  typename std::conditional<A8, ActX<kFfnThreads, (NS + 1) / 2>, char>::type XV;
  if constexpr (A8) act_x_load(a.x, a.H, XV);
  const int wave = threadIdx.x / kWave;
  if constexpr (FMT == WFMT_FP8_B128 && !A8 && !AW) resident_priority(a);
  if constexpr (FMT == WFMT_FP8_B128 && !A8 && !AW) {
    const int NW = gridDim.x * kFfnWaves;
    if (a.M == 1 && a.has_shared && a.I <= NW && a.S * a.I >= NW) {
      gateup_shared_first<NS>(a, QL.bits[wave], QL.base[wave], blockIdx.x * kFfnWaves + wave, NW);
      return;
    }
  }
  WaveQueue Q;
  gateup_queue(a, Q, QL.bits[wave], QL.base[wave], SEL);
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
  __shared__ int SEL[kMaxPairs];
  const int wave = threadIdx.x / kWave;
  WaveQueue Q;
  tokens_queue<NWV>(a, Q, QL.bits[wave], QL.base[wave], SEL);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  gateup_tokens<FMT, NS, UPG, true, false, AW>(a, Q, QL.cnt[wave], &QL.next, blockIdx.x,
                                               gridDim.x);
}

// gate/up with several tokens whose activations fit the LDS copy (M * H * 2 <= kXlBytes): one
// workgroup of TPB threads per CU stages every token's x in LDS and its waves take UPG units at
// a time from an LDS counter (gateup_xl_range).
template <int FMT, int NS, int UPG, int TPB>
__global__ __launch_bounds__(TPB) void gateup_xl_kernel(FfnArgs a) {
  constexpr int NWV = TPB / kWave;
  __shared__ QueueLdsT<NWV> QL;
  __shared__ int SEL[kMaxPairs];
  __shared__ uint4 XL[kXlBytes / 16];
  const int wave = threadIdx.x / kWave;
  xl_stage<FMT, TPB>(a, XL);
  WaveQueue Q;
  tokens_queue<NWV>(a, Q, QL.bits[wave], QL.base[wave], SEL);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  constexpr int kAlign = UPG == 2 ? ~1 : ~0;
  WaveBalance B;
  wave_balance_build(B, Q, QL.cnt[wave], a.I, kUnitCost, kPairCost);
  const int u0 = wave_balance_unit(B, (int64_t)B.total * blockIdx.x / gridDim.x) & kAlign;
  const int u1 = wave_balance_unit(B, (int64_t)B.total * (blockIdx.x + 1) / gridDim.x) & kAlign;
  if (threadIdx.x == 0) QL.next = u0;
  __syncthreads();  // the counter, and the staged activations
  gateup_xl_range<FMT, NS, UPG>(a, Q, &QL.next, u1, XL);
}

// down projection of the units of the workgroup / wave split (down_rows_range).
template <int FMT, int NS2, int RPW2, bool DYN, int TPB, bool A8, bool AW = false>
__global__ __launch_bounds__(TPB) void down_kernel(FfnArgs a) {
  constexpr int NWV = TPB / kWave;
  __shared__ QueueLdsT<NWV> QL;
  const int wave = threadIdx.x / kWave;
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int part = DYN ? (int)blockIdx.x : (int)blockIdx.x * NWV + wave;
  const int nparts = DYN ? (int)gridDim.x : (int)gridDim.x * NWV;
  const int units_per_expert = a.H / RPW2;
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
  NoReport rep;
  down_rows_range<FMT, NS2, RPW2, DYN, A8, AW>(a, Q, &QL.next, v0, v1, rep);
}

// down projection over flattened rows (down_flat_range), per-wave split.
template <int FMT, int C2G, int NSU, int GB, bool A8>
__global__ __launch_bounds__(kFfnThreads) void down_flat_kernel(FfnArgs a) {
  constexpr int R = kWave * NSU / C2G;
  __shared__ QueueLds QL;
  const int wave = threadIdx.x / kWave;
  if constexpr (FMT == WFMT_FP8_B128 && !A8) resident_priority(a);
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int gw = blockIdx.x * kFfnWaves + wave;
  const int NW = gridDim.x * kFfnWaves;
  const int upe = a.H / R;
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
  NoReport rep;
  down_flat_range<FMT, C2G, NSU, GB, A8>(a, Q, v0, v1, rep);
}

// down projection over flattened rows with several tokens: each resident workgroup of TPB
// threads (one per CU at these sizes) takes a cost-weighted range (a unit costs one pass per
// pair) and its waves take units one at a time from an LDS counter, so that a CU's waves end
// together; every lane is busy whatever the row length (the row-chunk kernel idles 16 of 64
// lanes on the 48-chunk MXFP4 rows of intermediate 1536).  AL holds each wave's first-pair row
// of a (down_flat_dyn).
template <int FMT, int C2G, int NSU, int GB, int TPB>
__global__ __launch_bounds__(TPB) void down_flat_cu_kernel(FfnArgs a) {
  constexpr int R = kWave * NSU / C2G;
  constexpr int NWV = TPB / kWave;
  __shared__ QueueLdsT<NWV> QL;
  __shared__ float AL[NWV][C2G * Gran<FMT, GB>::kVals];
  const int wave = threadIdx.x / kWave;
  WaveQueue Q;
  wave_queue_build(Q, QL.bits[wave], QL.base[wave], a.ids, a.M * a.S, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  const int upe = a.H / R;
  WaveBalance B;
  wave_balance_build(B, Q, QL.cnt[wave], upe, kUnitCost, kPairCost);
  const int v0 = wave_balance_unit(B, (int64_t)B.total * blockIdx.x / gridDim.x);
  const int v1 = wave_balance_unit(B, (int64_t)B.total * (blockIdx.x + 1) / gridDim.x);
  if (threadIdx.x == 0) QL.next = v0;
  __syncthreads();
  down_flat_dyn<FMT, C2G, NSU, GB>(a, Q, v1, &QL.next, AL[wave]);
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

template <int FMT, int NS, int UPG, int TPB>
hipError_t launch_gateup_xl_t(const FfnArgs& a, hipStream_t stream) {
  static int grid = 0;
  auto kern = gateup_xl_kernel<FMT, NS, UPG, TPB>;
  hipError_t err = resident_grid(kern, &grid, TPB);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(TPB), 0, stream, a);
  return hipGetLastError();
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
    // Past the chunk counts whose registers allow three waves per SIMD with the activations in
    // registers, the activations go to LDS where they fit, at four waves per SIMD (8-layer 1T
    // stack, 4 tokens: 158 -> 155 us per layer; at the smaller chunk counts it gained nothing).
    constexpr bool kWide = NS <= (FMT == WFMT_FP8_B128 ? 5 : 3);
    if (!kWide && a.M > 1 && (int64_t)a.M * a.H * 2 <= kXlBytes)
      return launch_gateup_xl_t<FMT, NS, 1, 1024>(a, stream);
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

template <int FMT, int C2G, int NSU, int GB, int TPB>
hipError_t launch_down_flat_cu_t(const FfnArgs& a, hipStream_t stream) {
  static int grid = 0;
  auto kern = down_flat_cu_kernel<FMT, C2G, NSU, GB, TPB>;
  hipError_t err = resident_grid(kern, &grid, TPB);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(TPB), 0, stream, a);
  return hipGetLastError();
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
  if (a.M > 1) {
    if (wfmt == WFMT_MXFP4 && a.I == 1536 && a.H % 8 == 0)
      return launch_down_flat_cu_t<WFMT_MXFP4, 96, 12, 8, kCuThreadsWide>(a, stream);
    return hipErrorNotSupported;
  }
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
  return launch_combine(a, stream);
}

hipError_t launch_combine(const FfnArgs& a, hipStream_t stream) {
  const int n = a.M * a.H;
  if (a.residual)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((n + 255) / 256), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((n + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
