// Internal launchers of the gfx950 kernels; the C ABI (capi.cpp) validates arguments and calls
// these.  Everything here is enqueue-only: no allocation, no host synchronization.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Counter words at the start of the workspace (zero between calls; each call restores zero).
constexpr int kCounterWords = 1024;

hipError_t launch_quant_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* s, int32_t* nonfinite, hipStream_t stream);
hipError_t launch_quant_fp8(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s,
                            int32_t* nonfinite, hipStream_t stream);

struct RouteArgs {
  const uint16_t* x;   // [M][H] bf16
  const float* wr;     // [E][H]
  const float* bias;   // [E] or null
  double* logits;      // [M][E]
  int32_t* ids;        // [M][S]
  float* w;            // [M][S]
  int M, H, E, k, has_shared;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

// Kernel arguments of the expert FFN (passed by value).
struct FfnArgs {
  const uint8_t* w13;
  const void* w13s;
  const uint8_t* w2;
  const void* w2s;
  const uint16_t* x;
  const int32_t* ids;
  const float* topk_w;
  float* a_buf;       // [M*S][I] fp32
  float* o_buf;       // [M*S][H] fp32
  uint16_t* y;
  int32_t* status;
  int M, S, H, I, n_experts;
};

int ffn_chunks_per_lane(int wfmt, int K);
// gate/up + SwiGLU into a_buf; then down projection + weighted combine into y.
hipError_t launch_gate_up(const FfnArgs& a, int wfmt, hipStream_t stream);
hipError_t launch_down_combine(const FfnArgs& a, int wfmt, hipStream_t stream);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

}  // namespace moe
