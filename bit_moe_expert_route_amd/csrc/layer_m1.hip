// One token's whole MoE layer in one launch: router logits, expert selection, gate/up + SwiGLU,
// down projection and the weighted combine (plus the residual in the layer stack).
//   molayo1419.me Xiaomi 1T page, section 1: at batch 1 the time goes to the gaps between
//   operators (launches, synchronizations, round trips through global memory) as much as to the
//   operators, which is why the page's engine keeps one persistent kernel per step; section 2:
//   expert FFN weights in MXFP4.
//   blogs.novita.ai "Optimizing GLM4-MoE for production", section 1: the shared expert runs as
//   one more slot of the fused MoE; since it does not depend on the routing it can start first.
//
// Work of the resident grid (NW waves, all resident at once):
//   1. Workgroups [0, L) compute the router logits, one expert per workgroup (the arithmetic of
//      the logits kernel, so the logits and the selection are bit-identical to the staged path);
//      meanwhile the other waves stream the shared expert's gate/up units, which need no
//      routing.
//   2. Every wave waits for the logits, selects the token's experts itself and takes its share
//      of the routed gate/up units.  The shares are balanced: a logits wave's share is smaller
//      by the logits' cost, a shared-expert wave's by its shared units.
//   3. Every wave takes its share of the down units (expert-major), loading an expert's a as
//      soon as all of it is there.
//   4. The wave that finishes the last expert's last unit of a 64-row block sums the S slot
//      outputs of those rows in slot order once they are all there, and stores y (the combine
//      kernel's arithmetic, so y is bit-identical too).
// Hand-offs carry the call's epoch with every value (LaunchIO): a consumer reloads until what it
// needs is from this call.  There is no atomic read-modify-write, counter, fence, reset or
// grid-wide barrier: per-call work of a contended atomic serializes (about 20 ns each), which
// thousands of waves cannot afford.  The epoch is one more than the call count of the
// workgroup's own counter word, which every workgroup of a call advances for its residue class
// of the kMaxGrid words, so all workgroups of a call agree on it whatever the grid size of the
// calls before.
#include "ffn_body.h"
#include "route_select.h"

namespace moe {
namespace {

// Words of the workspace's counter area used by the layer.
constexpr int kMaxGrid = 2048;              // call counters, one per workgroup slot
constexpr int kLogitStamp = kMaxGrid;       // [kMaxExperts]: logits workgroup b done (epoch)
static_assert(kLogitStamp + kMaxExperts <= kCounterWords, "counter area too small");
constexpr int kRowBlock = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x % kWave; }

// Wait until this wave's memory operations have completed (its relaxed atomic stores are then
// visible device-wide); the compiler may not move memory accesses across it.
__device__ __forceinline__ void vmem_drain() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
}

// Wait until the L logits workgroups have stamped their logits with the epoch (LP stamps per
// lane cover L <= 64 LP; every load is issued before any is checked).
template <int LP>
__device__ __forceinline__ void wait_logits(uint32_t* st, int L, const LaunchIO& io) {
  const int lane = lane_id();
  for (int it = 0;; ++it) {
    uint32_t v[LP];
#pragma unroll
    for (int j = 0; j < LP; ++j) {
      const int i = lane + kWave * j;
      v[j] = __hip_atomic_load(st + (i < L ? i : L - 1), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    bool ok = true;
#pragma unroll
    for (int j = 0; j < LP; ++j) ok = ok && v[j] == io.epoch;
    if (io.ready(ok, it)) break;
  }
  asm volatile("" ::: "memory");
}

// The down bodies' hook: the wave that finishes the last rank's last unit of a 64-row block
// combines that block once the wave's own units are done.
template <bool RES>
struct DownCombine {
  const FfnArgs* a;
  const LaunchIO* io;
  int rows;           // rows per down unit (divides 64)
  uint64_t slot_key;  // lane j < k: the logit key of slot j, for the weights
  int rb0 = 0, rb1 = 0;  // row blocks [rb0, rb1) to combine

  __device__ void unit_done(int q, int h0) {
    if (q == a->S - 1 && (h0 + rows) % kRowBlock == 0) {
      const int rb = h0 / kRowBlock;
      if (rb1 == rb0) rb0 = rb;
      rb1 = rb + 1;
    }
  }
  // y[h] = sum over slots j (in order) of w_j * o[j][h] for each block's 64 rows, one per lane
  __device__ void finish() {
    if (rb1 == rb0) return;
    const int lane = lane_id();
    const int S = a->S, H = a->H, k = a->k_routed;
    float w = select_weights(slot_key, k);
    if (S > k && lane == k) w = 1.0f;
    for (int rb = rb0; rb < rb1; ++rb) {
      const int h = rb * kRowBlock + lane;
      float ov[kMaxSlots];
      io->probe(a->o_buf, (int64_t)(S - 1) * H + h);
      for (int it = 0;; ++it) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j)
          ov[j] = io->get1(a->o_buf, (int64_t)(j < S ? j : 0) * H + h, ok);
        if (io->ready(ok, it)) break;
      }
      const uint16_t h_in = RES ? a->y[h] : 0;
      float y = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxSlots; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        const float nv = __builtin_fmaf(wj, ov[j], y);
        y = j < S ? nv : y;
      }
      if (RES)
        a->y[h] = f64_to_bf16(bf16_to_f64(h_in) + (double)y);
      else
        a->y[h] = f32_to_bf16(y);
    }
  }
};

// Down configurations: the flattened-row body (C2G granules of GB bytes per row, NSU granules
// per lane and unit) or the row-chunk body (NS2 16-byte chunks per lane, RPW2 rows per unit).
template <int C2G, int NSU, int GB>
struct DownFlat {
  static constexpr int kRows = kWave * NSU / C2G;
  template <int FMT, class Rep>
  __device__ static void run(const FfnArgs& a, const WaveQueue& Q, int v0, int v1, Rep& rep,
                             const LaunchIO& io) {
    down_flat_range<FMT, C2G, NSU, GB, false>(a, Q, v0, v1, rep, io);
  }
};
template <int NS2, int RPW2>
struct DownRows {
  static constexpr int kRows = RPW2;
  template <int FMT, class Rep>
  __device__ static void run(const FfnArgs& a, const WaveQueue& Q, int v0, int v1, Rep& rep,
                             const LaunchIO& io) {
    down_rows_range<FMT, NS2, RPW2, false, false, false>(a, Q, nullptr, v0, v1, rep, io);
  }
};

// Router logit of expert e for the one token, by the whole workgroup: the logits kernel's
// arithmetic (wave w takes the float4 chunks 64w + lane + 256j of Wr_e, an fp64 FMA chain per
// lane, the fixed-order DPP sum, then the 4 waves in order, then the bias).  Wave 0 stores it.
template <int NCH>
__device__ __forceinline__ void logit_of_expert(const RouteArgs& ra, int e, double* part) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int H = ra.H, nc = H / 4;
  int cc[NCH];
  bool cv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = wave * kWave + lane + kFfnThreads * j;
    cv[j] = c < nc;
    cc[j] = cv[j] ? c : nc - 1;
  }
  const float4* wr = reinterpret_cast<const float4*>(ra.wr + (int64_t)e * H);
  const uint2* xt = reinterpret_cast<const uint2*>(ra.x);
  float4 w4[NCH];
  uint2 xb[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) w4[j] = wr[cc[j]];
#pragma unroll
  for (int j = 0; j < NCH; ++j) xb[j] = xt[cc[j]];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    opaque(w4[j]);
    opaque(xb[j]);
    w4[j] = cv[j] ? w4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    xb[j] = cv[j] ? xb[j] : make_uint2(0, 0);
  }
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].x & 0xFFFF)), (double)w4[j].x, s);
    s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].x >> 16)), (double)w4[j].y, s);
    s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].y & 0xFFFF)), (double)w4[j].z, s);
    s = __fma_rn((double)bf16_to_f32((uint16_t)(xb[j].y >> 16)), (double)w4[j].w, s);
  }
  s = wave_sum_to_last(s);
  if (lane == kWave - 1) part[wave] = s;
  __syncthreads();
  if (wave == 0 && lane == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kFfnWaves; ++w) t += part[w];
    if (ra.bias) t += (double)ra.bias[e];
    __hip_atomic_store(reinterpret_cast<uint64_t*>(ra.logits + e),
                       (uint64_t)__double_as_longlong(t), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // part is reused by the next expert
}

// The wave's routing: selection over the logits (every wave), the grid's first wave also
// publishing ids and weights.
template <int KPER>
__device__ __forceinline__ void select_m1(const FfnArgs& a, const RouteArgs& ra, bool pub,
                                          int& id, uint64_t& key) {
  const int lane = lane_id();
  const int has_shared = a.S - a.k_routed;
  float w;
  wave_select<KPER, true>(ra.logits, a.E_routed, a.k_routed, has_shared, id, w, pub, &key);
  if (pub && lane < a.S) {
    a.ids_out[lane] = id;
    a.w_out[lane] = w;
  }
}

// Start of wave g's share of `total` units when the NL logits waves (first) carry a pre-cost of
// cl units each and the other NW - NL waves a pre-cost of cs units each: shares are balanced so
// that pre-cost + share is equal for all waves (an equal split when that would make a share
// negative).  Exact integer arithmetic, so neighbouring waves agree on their common boundary.
__device__ __forceinline__ int balanced_start(int g, int NW, int NL, int total, int cl_num,
                                              int cs_num, int cs_den) {
  // per-wave total T = (total + NL*cl + (NW-NL)*cs) / NW, with cs = cs_num / cs_den
  const int NS_ = NW - NL;
  const int64_t Tn = ((int64_t)total + (int64_t)NL * cl_num) * cs_den + (int64_t)NS_ * cs_num;
  const int64_t Td = (int64_t)NW * cs_den;                 // T = Tn / Td
  const int64_t shl_n = Tn - (int64_t)cl_num * Td;         // logits share * Td
  const int64_t shs_n = Tn * cs_den - (int64_t)cs_num * Td;  // shared share * Td * cs_den
  if (shl_n < 0 || shs_n < 0 || NS_ == 0) return (int)((int64_t)total * g / NW);
  if (g <= NL) return (int)((int64_t)g * shl_n / Td);
  return (int)(((int64_t)NL * shl_n * cs_den + (int64_t)(g - NL) * shs_n) / (Td * cs_den));
}

template <int FMT, int NS, class DC, bool RES>
__global__ __launch_bounds__(kFfnThreads, 2) void layer_m1_kernel(FfnArgs a, RouteArgs ra,
                                                               uint32_t* ctr) {
  constexpr int NCH = FMT == WFMT_FP8_B128 ? NS : 2 * NS;  // float4 chunks of Wr per thread
  __shared__ QueueLds QL;
  __shared__ double part[kFfnWaves];
  __shared__ uint32_t epoch_lds;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int G = gridDim.x, b = blockIdx.x;
  const int NW = G * kFfnWaves, g = b * kFfnWaves + wave;
  if (threadIdx.x == 0)
    epoch_lds = __hip_atomic_load(ctr + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  __syncthreads();
  const LaunchIO io{epoch_lds, a.status};
  const int E = a.E_routed, S = a.S, k = a.k_routed, I = a.I, H = a.H;
  const bool has_shared = S > k;
  const int L = E < G ? E : G;  // logits workgroups
  const bool pre_shared = has_shared && G > L;
  const int NL = L * kFfnWaves;
  // 1. logits, or the shared expert's gate/up units
  if (b < L) {
    for (int e = b; e < E; e += L) logit_of_expert<NCH>(ra, e, part);
    if (wave == 0) {
      vmem_drain();
      if (lane == 0)
        __hip_atomic_store(ctr + kLogitStamp + b, io.epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (pre_shared) {
    WaveQueue Qs;
    int v[kPairRegs];
    v[0] = lane == S - 1 ? E : -1;
#pragma unroll
    for (int j = 1; j < kPairRegs; ++j) v[j] = -1;
    wave_queue_from(Qs, QL.bits[wave], QL.base[wave], v, S, a.n_experts);
    const int gs = g - NL, NWs = NW - NL;
    const int u0 = (int)((int64_t)I * gs / NWs), u1 = (int)((int64_t)I * (gs + 1) / NWs);
    if constexpr (FMT == WFMT_MXFP4)
      gateup_one_token<FMT, NS>(a, Qs, u0, u1, io);
    else
      gateup_range<FMT, NS, 2, false, false, false>(a, Qs, nullptr, u0, u1, nullptr, nullptr,
                                                    io);
  }
  // 2. routing, then the routed gate/up units (all units when the shared ones were not taken)
  int id;
  uint64_t key;
  const int per = (E + kWave - 1) / kWave;
  const bool pub = g == 0;
  if (per <= 3) {
    wait_logits<3>(ctr + kLogitStamp, L, io);
    select_m1<3>(a, ra, pub, id, key);
  } else if (per <= 6) {
    wait_logits<6>(ctr + kLogitStamp, L, io);
    select_m1<6>(a, ra, pub, id, key);
  } else {
    constexpr int KP = (kMaxExperts + kWave - 2) / kWave;
    wait_logits<KP>(ctr + kLogitStamp, L, io);
    select_m1<KP>(a, ra, pub, id, key);
  }
  WaveQueue Q;
  {
    int v[kPairRegs];
    v[0] = id;
#pragma unroll
    for (int j = 1; j < kPairRegs; ++j) v[j] = -1;
    wave_queue_from(Q, QL.bits[wave], QL.base[wave], v, S, a.n_experts);
  }
  {
    const int total = (pre_shared ? k : S) * I;
    const int cl = (E + L - 1) / L;  // logits per logits workgroup, one unit of cost each
    const int u0 = pre_shared ? balanced_start(g, NW, NL, total, cl, I, NW - NL)
                              : (int)((int64_t)total * g / NW);
    const int u1 = pre_shared ? balanced_start(g + 1, NW, NL, total, cl, I, NW - NL)
                              : (int)((int64_t)total * (g + 1) / NW);
    if constexpr (FMT == WFMT_MXFP4)
      gateup_one_token<FMT, NS>(a, Q, u0, u1, io);
    else
      gateup_range<FMT, NS, 2, false, false, false>(a, Q, nullptr, u0, u1, nullptr, nullptr,
                                                    io);
  }
  // 3 + 4. down units of every expert; the blocks this wave closes are combined at its end
  {
    const int upe = H / DC::kRows;
    const int U = S * upe;
    const int v0 = (int)((int64_t)U * g / NW), v1 = (int)((int64_t)U * (g + 1) / NW);
    DownCombine<RES> rep{&a, &io, DC::kRows, key};
    DC::template run<FMT>(a, Q, v0, v1, rep, io);
  }
  // the next call's epoch: this workgroup advances its residue class of the counter words
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = b; i < kMaxGrid; i += G)
      __hip_atomic_store(ctr + i, io.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int NS, class DC, bool RES>
hipError_t launch_layer_m1_t(const FfnArgs& a, const RouteArgs& ra, uint32_t* ctr,
                             hipStream_t stream) {
  static int grid = 0;
  auto kern = layer_m1_kernel<FMT, NS, DC, RES>;
  hipError_t err = resident_grid(kern, &grid);
  if (err != hipSuccess) return err;
  if (grid > kMaxGrid) return hipErrorNotSupported;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kFfnThreads), 0, stream, a, ra, ctr);
  return hipGetLastError();
}

template <int FMT, int NS, class DC>
hipError_t launch_layer_m1_res(const FfnArgs& a, const RouteArgs& ra, uint32_t* ctr,
                               hipStream_t stream) {
  if (a.residual) return launch_layer_m1_t<FMT, NS, DC, true>(a, ra, ctr, stream);
  return launch_layer_m1_t<FMT, NS, DC, false>(a, ra, ctr, stream);
}

}  // namespace

// The one-launch layer exists for the shapes of the GLM-4.7 and 1T-class layers and their
// tensor-parallel ranks (hidden 5120 / 7168; intermediate 1536, 192, 2048, 256); other shapes
// return hipErrorNotSupported and take the staged launches.
hipError_t launch_layer_m1(const FfnArgs& a, const RouteArgs& ra, int wfmt, uint32_t* ctr,
                           hipStream_t stream) {
  if (a.M != 1 || a.logits == nullptr) return hipErrorNotSupported;
  if (wfmt == WFMT_FP8_B128 && a.H == 5120) {
    if (a.I == 1536) return launch_layer_m1_res<WFMT_FP8_B128, 5, DownFlat<192, 24, 8>>(a, ra, ctr, stream);
    if (a.I == 192) return launch_layer_m1_res<WFMT_FP8_B128, 5, DownFlat<24, 6, 8>>(a, ra, ctr, stream);
  } else if (wfmt == WFMT_MXFP4 && a.H == 5120) {
    if (a.I == 1536) return launch_layer_m1_res<WFMT_MXFP4, 3, DownFlat<96, 12, 8>>(a, ra, ctr, stream);
    if (a.I == 192) return launch_layer_m1_res<WFMT_MXFP4, 3, DownFlat<12, 3, 8>>(a, ra, ctr, stream);
  } else if (wfmt == WFMT_MXFP4 && a.H == 7168) {
    if (a.I == 2048) return launch_layer_m1_res<WFMT_MXFP4, 4, DownRows<1, 8>>(a, ra, ctr, stream);
    if (a.I == 256) return launch_layer_m1_res<WFMT_MXFP4, 4, DownFlat<16, 4, 8>>(a, ra, ctr, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace moe
