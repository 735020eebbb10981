// Pieces shared by the expert-FFN kernels: weight-format traits, block scale addressing,
// per-wave work-queue storage and the resident-grid size.
#pragma once
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kFfnThreads = 256;
constexpr int kFfnWaves = kFfnThreads / kWave;

template <int FMT>
struct Fmt;
template <>
struct Fmt<WFMT_FP8_B128> {
  static constexpr int kVals = 16;   // values per 16-byte chunk
  static constexpr int kXWords = 8;  // bf16 pairs per chunk
  __device__ static int64_t row_bytes(int K) { return K; }
};
template <>
struct Fmt<WFMT_MXFP4> {
  static constexpr int kVals = 32;
  static constexpr int kXWords = 16;
  __device__ static int64_t row_bytes(int K) { return K / 2; }
};

// FP8 block scales per row of blocks of a [R][K] matrix: ceil(K / 128) (the last block along K
// is partial when K is not a multiple of 128).
__device__ __forceinline__ int fp8_blocks(int K) { return (K + 127) >> 7; }

// Raw block scale of chunk c of row r of one expert matrix [R][K] (fp32 bits for FP8, the
// E8M0 byte for MXFP4).  Decoding waits until the chunk is consumed, so a scale never stalls
// the loads behind it.
template <int FMT>
__device__ __forceinline__ uint32_t scale_raw(const void* scales, int K, int r, int c) {
  if constexpr (FMT == WFMT_FP8_B128)
    return reinterpret_cast<const uint32_t*>(scales)[(r >> 7) * fp8_blocks(K) + (c >> 3)];
  else
    return reinterpret_cast<const uint8_t*>(scales)[(int64_t)r * (K >> 5) + c];
}

template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t raw) {
  if constexpr (FMT == WFMT_FP8_B128) return __uint_as_float(raw);
  else return e8m0_to_f32(raw);
}

// Scale elements of one expert matrix [R][K].
template <int FMT>
__device__ __forceinline__ int64_t scale_elems(int R, int K) {
  return FMT == WFMT_FP8_B128 ? (int64_t)fp8_blocks(R) * fp8_blocks(K) : (int64_t)R * (K >> 5);
}

template <int FMT>
__device__ __forceinline__ const void* scale_ptr(const void* base, int64_t elems_before) {
  if constexpr (FMT == WFMT_FP8_B128) return reinterpret_cast<const float*>(base) + elems_before;
  else return reinterpret_cast<const uint8_t*>(base) + elems_before;
}

// Per-wave queue storage in LDS for NWV waves, and the workgroup's unit counter.
template <int NWV>
struct QueueLdsT {
  uint32_t bits[NWV][kBitmapWords];
  int base[NWV][kBitmapWords];
  int cnt[NWV][kMaxPairs];
  int next;
};
using QueueLds = QueueLdsT<kFfnWaves>;

// Unit costs for the cost-weighted split: a unit's first pair (weights from HBM, activations in
// registers) counts kUnitCost, every further pair (activations reloaded from L2) kPairCost.
// Measured on the 4- and 16-token layers, a further pair costs about as much as the first.
constexpr int kUnitCost = 1;
constexpr int kPairCost = 1;

// Kernels balanced within a CU run one workgroup of kCuThreads (or kCuThreadsWide when the
// kernel's registers allow three waves per SIMD) per CU.  Waves of a CU are not served alike:
// measured on the gate/up and down kernels, the waves of a CU's first-resident workgroup ended
// 2-5 us before those of the later ones for the same work.  With one workgroup per CU its waves
// take units from an LDS counter, so a CU's waves finish within one step of each other.
constexpr int kCuThreads = 512;
constexpr int kCuThreadsWide = 768;

// Raw buffer descriptors: word 3 with the 32-bit data format that untyped buffer loads take,
// and the nt bit of a buffer load's cache-policy operand.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

// A buffer descriptor over the n bytes at p (p wave-uniform); loads past n return zero without
// touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, kRsrcWord3);
}

// Persistent grid: resident workgroups per CU (occupancy, at most kMaxWgPerCu) times CUs.
constexpr int kMaxWgPerCu = 4;

template <typename K>
hipError_t resident_grid(K kern, int* cache, int threads = kFfnThreads) {
  if (*cache > 0) return hipSuccess;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  *cache = (per_cu < kMaxWgPerCu ? per_cu : kMaxWgPerCu) * cus;
  return hipSuccess;
}

}  // namespace
}  // namespace moe
