// Internal launchers of the gfx950 kernels; the C ABI (capi.cpp) validates arguments and calls
// these.  Everything here is enqueue-only: no allocation, no host synchronization.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_quant_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* s, int32_t* nonfinite, hipStream_t stream);
hipError_t launch_quant_fp8(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s,
                            int32_t* nonfinite, hipStream_t stream);

hipError_t launch_route(const uint16_t* x, int M, int H, const float* wr, const float* bias,
                        int E, int k, int has_shared, int32_t* ids, float* w, double* logits,
                        hipStream_t stream);

// Kernel arguments of the expert FFN phases (passed by value).
struct FfnArgs {
  const uint8_t* w13;
  const void* w13s;
  const uint8_t* w2;
  const void* w2s;
  const uint16_t* x;
  const int32_t* ids;
  const float* topk_w;
  float* a_buf;  // [M*S][I] fp32
  float* o_buf;  // [M*S][H] fp32
  uint16_t* y;
  int32_t* status;
  int M, S, H, I, n_experts;
  int ib, hb, items13, items2, tg13, tg2;
};

// Launch shape of the FFN phases for one problem shape.
struct FfnPlan {
  int ns13, ns2;          // 16-byte chunks per lane per row (gate/up, down)
  int max_active;         // upper bound on distinct experts
  int ib, hb;             // rows per item
  int items13, items2;    // items per expert
  int tg13, tg2;          // tokens staged in LDS at a time
  size_t lds13, lds2;     // dynamic LDS bytes
};

FfnPlan plan_ffn(int wfmt, int M, int S, int H, int I, int n_experts);
hipError_t launch_ffn(const FfnArgs& a, const FfnPlan& p, int wfmt, hipStream_t stream);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

}  // namespace moe
