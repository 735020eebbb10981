// Internal launchers of the gfx950 kernels; the C ABI (capi.cpp) validates arguments and calls
// these.  Everything here is enqueue-only: no allocation, no host synchronization.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Counter words at the start of the workspace (zero-filled once; the one-token one-launch layer
// keeps its per-call counters and stamps there).
constexpr int kCounterWords = 4096;

hipError_t launch_quant_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* s, int32_t* nonfinite, hipStream_t stream);
hipError_t launch_quant_fp8(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s,
                            int32_t* nonfinite, hipStream_t stream);

struct RouteArgs {
  const uint16_t* x;   // [M][H] bf16: the router input, or the residual stream h with gamma set
  const float* wr;     // [E][H]
  const float* bias;   // [E] or null
  double* logits;      // [M][E]
  int32_t* ids;        // [M][S]
  float* w;            // [M][S]
  // RMSNorm (launch_rmsnorm): xn_out = bf16((x * r) * gamma), r = 1/sqrt(mean(x^2) + eps) in
  // fp64; x_copy (nullable) receives a copy of x.
  const float* gamma;
  double eps;
  uint16_t* xn_out;
  uint16_t* x_copy;
  int M, H, E, k, has_shared;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);
hipError_t launch_logits_only(const RouteArgs& a, hipStream_t stream);
hipError_t launch_rmsnorm(const RouteArgs& a, hipStream_t stream);

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
  uint16_t* y;        // output [M][H] bf16; with residual set, y is the residual stream h and
  bool residual;      // the combine writes h = bf16(h + sum_j w_j o_j) in place
  int32_t* status;
  int M, S, H, I, n_experts;
  int has_shared;  // 1: expert n_experts - 1 is a shared expert, in every token's last slot
  int cus;         // the device's compute units (0: unknown): a resident grid's workgroups
                   // below it are the first ones on their CUs
  // Selection in the gate/up kernel: with logits set ([M][E_routed] fp64) the kernel selects the
  // tokens' experts itself (the router's rule) instead of reading ids, and its first workgroup
  // writes ids_out / w_out [M][S] for the kernels that follow.  One token: every wave selects;
  // several: the waves of each workgroup share the tokens and the ids through LDS.
  const double* logits;
  int32_t* ids_out;
  float* w_out;
  int E_routed, k_routed;
  // W8A8 with several tokens (workspace): x quantized to bf16 code values [M][H] with block
  // scales [M][H/128]; a_buf quantized to fp32 code values aq [M*S][I], scales [M*S][I/128]
  uint16_t* xq;
  float* x_scales;
  float* aq;
  float* a_scales;
};

int ffn_chunks_per_lane(int wfmt, int K);
// gate/up + SwiGLU into a_buf; then down projection + weighted combine into y.
hipError_t launch_gate_up(const FfnArgs& a, int wfmt, hipStream_t stream);
hipError_t launch_down_combine(const FfnArgs& a, int wfmt, hipStream_t stream);
// gate/up with several tokens on the matrix cores for the experts with 2..16 pairs, the others
// on the vector path, in one launch (ffn_mfma.hip); hipErrorNotSupported where it has no form
// (one token, other formats), for launch_gate_up to take.
hipError_t launch_gate_up_mfma(const FfnArgs& a, int wfmt, hipStream_t stream);
// down projection + combine, likewise (MXFP4 with intermediate 256, 384, 1536 or 2048).
hipError_t launch_down_mfma(const FfnArgs& a, int wfmt, hipStream_t stream);
// the weighted combine of the slot outputs into y (with the residual when a.residual)
hipError_t launch_combine(const FfnArgs& a, hipStream_t stream);

// One token's whole layer in one launch (layer_m1.hip): the router's logits and selection (a
// with logits, ids_out, w_out, E_routed, k_routed set as for the selecting gate/up kernel), the
// expert FFN and the combine (with the residual when a.residual).  a.a_buf and a.o_buf are
// 64-bit words [S][I] and [S][H] (value and call epoch); ctr: the workspace's counter words.
// hipErrorNotSupported for the shapes it is not built for.
hipError_t launch_layer_m1(const FfnArgs& a, const RouteArgs& ra, int wfmt, uint32_t* ctr,
                           hipStream_t stream);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// Verify-acceptance of one speculative block (verify.hip).  Workspace pieces: st (st[0]: the
// rejected position of the current sampling call), then per (row, chunk) cm / ca / cs, per row
// (m, Z), per chunk of one row the residual mass.  Nothing carries over between calls.
struct VerifyArgs {
  const float* L;        // [K+1][V] target logits
  const float* Q;        // [K][V] draft probabilities, or null (greedy)
  const int32_t* d;      // [K] draft tokens
  const float* u;        // [K+1] uniforms in [0, 1) (sampling)
  int32_t* out;          // [K+1] accepted tokens, then the drawn one
  int32_t* count;        // [1] number of tokens written
  uint32_t* st;          // [4]
  float* cm;             // [K+1][nch] chunk max
  int32_t* ca;           // [K+1][nch] chunk argmax (lowest index)
  double* cs;            // [K+1][nch] chunk sum of exp(l - chunk max)
  double* rowmz;         // [K+1][2] row max, row sum of exp(l - max)
  double* rmass;         // [nch] residual mass per chunk of the rejected row
  int K, V, nch;
};
int verify_chunks(int V);

// Fused QK-norm + RoPE (qk_rope.hip), in place on qk.
struct QkRopeArgs {
  uint16_t* qk;           // token t's heads at qk + t * stride: nq query heads, then nk key heads
  const int32_t* pos;     // [M]
  const float* gamma_q;   // [hd]
  const float* gamma_k;   // [hd]
  double eps, theta;
  int64_t stride;
  int M, nq, nk, hd, rot;
};
hipError_t launch_qk_norm_rope(const QkRopeArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, bool vec, hipStream_t stream);

}  // namespace moe
