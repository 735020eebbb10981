// One token's expert selection by one wave: the router's top-k rule, shared by the top-k
// kernel and the gate/up kernels (which select in their prologue instead of waiting for a top-k
// launch: with one token every wave, with several the waves of each workgroup in turn).
//   blogs.novita.ai "Optimizing GLM4-MoE for production", section 1: top 9 of 161, the shared
//   expert always last; molayo1419.me Xiaomi 1T page, section 1: sparse top-k routing.
// Experts ranked by (fp64 logit descending, index ascending); the k best get
// w = sigmoid(l) / (sum of the k sigmoids, in slot order), rounded once to fp32; with a shared
// expert, slot k is id E with weight 1.
#pragma once
#include <type_traits>

#include "moe_device.h"

namespace moe {
namespace {

// Lane l holds the order-preserving keys of experts l + 64r (r < KPER, KPER * 64 >= E) and
// tracks its best (largest key, lowest index).  Each round takes the wave maximum as a 32-bit
// DPP maximum of the high words, then, only when several lanes hold that high word, a second
// one of their low words; the winner is the only lane holding the maximum, else the lowest
// index among the holders; the winner then drops that key.  On return lane j < k + has_shared
// holds slot j's id and (with weights set; wave-uniform) its weight; other lanes hold id -1.
// Weights of the k selected experts from their keys (lane j < k holds slot j's key): sigmoid
// per slot in its lane, the sum in slot order, each weight rounded once to fp32.  Lanes >= k
// return 0.
__device__ __forceinline__ float select_weights(uint64_t my_key, int k) {
  const int lane = threadIdx.x % kWave;
  const double sg = (lane < k) ? 1.0 / (1.0 + exp(-f64_from_key(my_key))) : 0.0;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += read_lane(sg, j);
  return (lane < k) ? __double2float_rn(sg / sum) : 0.0f;
}

struct NoPrefetch {
  __device__ void operator()() const {}
};

// COHERENT: the logits were written by other waves of the same launch and are read with
// device-scope atomic loads.  slot_key (nullable) receives slot j's key in lane j < k, from which
// select_weights gives the weights later.  pre() issues further loads right behind the logits'
// (none by default): loads issued later, so waiting for the logits leaves them in flight.
template <int KPER, bool COHERENT = false, class Pre = NoPrefetch>
__device__ __forceinline__ void wave_select(const double* lt, int E, int k, int has_shared,
                                            int& slot_id, float& slot_w, bool weights = true,
                                            uint64_t* slot_key = nullptr, const Pre& pre = Pre()) {
  const int lane = threadIdx.x % kWave;
  double lv[KPER];
#pragma unroll
  for (int r = 0; r < KPER; ++r) {
    const int ee = lane + kWave * r;
    const double* src = lt + (ee < E ? ee : E - 1);
    if constexpr (COHERENT)
      lv[r] = __longlong_as_double((long long)__hip_atomic_load(
          reinterpret_cast<uint64_t*>(const_cast<double*>(src)), __ATOMIC_RELAXED,
          __HIP_MEMORY_SCOPE_AGENT));
    else
      lv[r] = *src;
  }
  if constexpr (!std::is_same<Pre, NoPrefetch>::value) {
    __builtin_amdgcn_sched_barrier(0);
    pre();
    __builtin_amdgcn_sched_barrier(0);
  }
  uint64_t key[KPER];
#pragma unroll
  for (int r = 0; r < KPER; ++r) {
    opaque(lv[r]);
    const uint64_t kv = f64_key(lv[r]);
    key[r] = lane + kWave * r < E ? (kv > 1ull ? kv : 1ull) : 0ull;  // 0: absent or taken
  }
  auto lane_best = [&](uint64_t& best, int& bidx) {
    best = key[0];
    bidx = lane;
#pragma unroll
    for (int r = 1; r < KPER; ++r) {
      const bool gt = key[r] > best;
      best = gt ? key[r] : best;
      bidx = gt ? lane + kWave * r : bidx;
    }
  };
  uint64_t best;
  int bidx;
  lane_best(best, bidx);
  uint64_t my_key = 0;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t mh = wave_max_u32((uint32_t)(best >> 32));
    const uint64_t hh = __ballot((uint32_t)(best >> 32) == mh);
    // the low word decides only when several lanes hold the high word
    const uint32_t ml =
        (hh & (hh - 1)) == 0
            ? (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, __builtin_ctzll(hh))
            : wave_max_u32((uint32_t)(best >> 32) == mh ? (uint32_t)best : 0u);
    const uint64_t kmax = ((uint64_t)mh << 32) | ml;
    const uint64_t hit = __ballot(best == kmax);
    int idx;
    if ((hit & (hit - 1)) == 0)
      idx = __builtin_amdgcn_readlane(bidx, __builtin_ctzll(hit));
    else
      idx = (int)wave_min_u32(best == kmax ? (uint32_t)bidx : 0xFFFFFFFFu);
    if (lane == (idx & (kWave - 1))) {
#pragma unroll
      for (int r = 0; r < KPER; ++r)
        if (r == idx / kWave) key[r] = 0;
    }
    lane_best(best, bidx);
    if (lane == j) { my_key = kmax; my_i = idx; }
  }
  slot_id = -1;
  slot_w = 0.0f;
  if (lane < k) slot_id = my_i;
  if (slot_key) *slot_key = my_key;
  if (weights) slot_w = select_weights(my_key, k);
  if (has_shared && lane == k) {
    slot_id = E;
    slot_w = 1.0f;
  }
}

// Several tokens by the NWV waves of one workgroup: wave w selects tokens w, w + NWV, ... over
// their logits [M][E] with wave_select; slot j of token t goes to sel[t * S + j] and, when pub,
// to ids_out / w_out as well.  The caller meets a workgroup barrier before reading sel.
template <int NWV>
__device__ __forceinline__ void select_tokens(const double* logits, int M, int E, int k,
                                              int has_shared, int* sel, bool pub,
                                              int32_t* ids_out, float* w_out) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int S = k + has_shared, per = (E + kWave - 1) / kWave;
  for (int t = wave; t < M; t += NWV) {
    const double* lt = logits + (int64_t)t * E;
    int id;
    float w;
    if (per <= 3)
      wave_select<3>(lt, E, k, has_shared, id, w, pub);
    else if (per <= 6)
      wave_select<6>(lt, E, k, has_shared, id, w, pub);
    else
      wave_select<(kMaxExperts + kWave - 1) / kWave>(lt, E, k, has_shared, id, w, pub);
    if (lane < S) {
      sel[t * S + lane] = id;
      if (pub) {
        ids_out[t * S + lane] = id;
        w_out[t * S + lane] = w;
      }
    }
  }
}

}  // namespace
}  // namespace moe
