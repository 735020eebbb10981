// C ABI of the MoE decode layer: host-side validation, workspace carving and kernel launches.
// Nothing here allocates device memory or synchronizes the host.
#include "moe_mx.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kCounterBytes = moe::kCounterWords * sizeof(int32_t);

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Shape checks shared by every call (pointers are checked per call).
moe_status check_shape(const moe_layer* L) {
  if (!L) return MOE_ERR_INVALID;
  if (L->wfmt != MOE_WFMT_MXFP4 && L->wfmt != MOE_WFMT_FP8_B128 &&
      L->wfmt != MOE_WFMT_FP8_B128_A8)
    return MOE_ERR_INVALID;
  // hidden: whole 128-wide blocks for both formats; inter: whole 32-value MX blocks for MXFP4
  // and a multiple of 32 for FP8 too (a tensor-parallel shard's intermediate slice, e.g. 192 of
  // 1536: the FP8 block scales' last 128-block along the intermediate axis is then partial)
  if (L->hidden <= 0 || L->inter <= 0 || L->hidden % 128 || L->inter % 32)
    return MOE_ERR_INVALID;
  // W8A8 quantizes the activations in whole 128-value blocks along K
  if (L->wfmt == MOE_WFMT_FP8_B128_A8 && L->inter % 128) return MOE_ERR_UNSUPPORTED;
  // The router gives each thread at most 8 float4 chunks of a row (hidden <= 8192); the expert
  // kernels give each lane at most 4 16-byte chunks of a down row (inter <= 4096 / 8192 for
  // FP8 / MXFP4).
  const int32_t vals = (L->wfmt == MOE_WFMT_MXFP4) ? 32 : 16;
  if (L->hidden > 8192 || L->inter > 4 * 64 * vals) return MOE_ERR_UNSUPPORTED;
  if (L->n_routed < 1 || L->n_routed > MOE_MAX_EXPERTS) return MOE_ERR_INVALID;
  if (L->has_shared != 0 && L->has_shared != 1) return MOE_ERR_INVALID;
  if (L->top_k < 1 || L->top_k > L->n_routed) return MOE_ERR_INVALID;
  if (L->top_k + L->has_shared > MOE_MAX_SLOTS) return MOE_ERR_INVALID;
  return MOE_OK;
}

moe_status check_experts(const moe_layer* L) {
  if (!L->w13 || !L->w13_scale || !L->w2 || !L->w2_scale) return MOE_ERR_INVALID;
  if (!aligned(L->w13, 16) || !aligned(L->w2, 16) || !aligned(L->w13_scale, 16) ||
      !aligned(L->w2_scale, 16))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

struct WsLayout {
  size_t counters, logits, a_buf, o_buf, xn, ids, w, xq, x_scales, aq, a_scales, a64, o64, total;
};

WsLayout layout(const moe_layer* L, int32_t M) {
  const size_t S = (size_t)L->top_k + L->has_shared;
  WsLayout w;
  size_t off = 0;
  w.counters = off;
  off += align_up(kCounterBytes);
  w.logits = off;
  off += align_up((size_t)M * L->n_routed * sizeof(double));
  w.a_buf = off;
  off += align_up((size_t)M * S * L->inter * sizeof(float));
  w.o_buf = off;
  off += align_up((size_t)M * S * L->hidden * sizeof(float));
  // layer stack: normalized activations and the routing of the current layer
  w.xn = off;
  off += align_up((size_t)M * L->hidden * sizeof(uint16_t));
  w.ids = off;
  off += align_up((size_t)M * S * sizeof(int32_t));
  w.w = off;
  off += align_up((size_t)M * S * sizeof(float));
  // W8A8 with several tokens: the quantized activations and their block scales
  w.xq = off;
  off += align_up((size_t)M * L->hidden * sizeof(uint16_t));
  w.x_scales = off;
  off += align_up((size_t)M * (L->hidden / 128) * sizeof(float));
  w.aq = off;
  off += align_up((size_t)M * S * L->inter * sizeof(float));
  w.a_scales = off;
  off += align_up((size_t)M * S * (L->inter / 128 + 1) * sizeof(float));
  // the one-token one-launch layer: a and o of every slot as (value, call epoch) words
  w.a64 = off;
  off += align_up(S * L->inter * sizeof(uint64_t));
  w.o64 = off;
  off += align_up(S * L->hidden * sizeof(uint64_t));
  w.total = off;
  return w;
}

moe_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws || !aligned(ws, kAlign)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

inline moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status layer_decode_impl(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                             int32_t* topk_ids, float* topk_w, double* logits_out,
                             uint16_t* y_bf16, void* ws, size_t ws_bytes, int32_t* dev_status,
                             bool one_launch, hipStream_t stream);

// The library-owned workspace of moe_layer_decode_static: one copy per GPU, held until the
// process ends.  In host code `scratch` only names the symbol; its device address on the
// current GPU comes from hipGetSymbolAddress, once per device, and is the only form of it that
// host code hands to kernels or fills.
__device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address.  On the first call on a device the address is looked
// up and the counter area (the part that must start at zero, as in a fresh workspace) is
// cleared by the fill kernel on `stream`, ahead of the call's own kernels.
moe_status static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    if (moe::launch_fill_zero(ptr, kCounterBytes, stream) != hipSuccess) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_workspace_bytes(const moe_layer* layers, int32_t n_layers, int32_t M) {
  if (!layers || n_layers < 1 || M < 1 || M > MOE_MAX_TOKENS) return 0;
  size_t need = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    if (check_shape(&layers[l]) != MOE_OK) return 0;
    const size_t t = layout(&layers[l], M).total;
    if (t > need) need = t;
  }
  return need;
}

// Verify workspace: the decision word, then per (row, chunk) the chunk max, argmax and exp-sum,
// the per-row (max, sum), and the per-chunk residual mass; each piece 256-aligned.
struct VerifyLayout {
  size_t st, cm, ca, cs, rowmz, rmass, total;
};

static size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

static VerifyLayout verify_layout(int32_t K, int32_t V) {
  const size_t nch = (size_t)moe::verify_chunks(V), rows = (size_t)K + 1;
  VerifyLayout l{};
  size_t off = 0;
  l.st = off; off += up256(4 * sizeof(uint32_t));
  l.cm = off; off += up256(rows * nch * sizeof(float));
  l.ca = off; off += up256(rows * nch * sizeof(int32_t));
  l.cs = off; off += up256(rows * nch * sizeof(double));
  l.rowmz = off; off += up256(2 * rows * sizeof(double));
  l.rmass = off; off += up256(nch * sizeof(double));
  l.total = off;
  return l;
}

static bool verify_shape_ok(int32_t K, int32_t V) {
  return K >= 0 && K < MOE_MAX_TOKENS && V >= 1 && V <= MOE_MAX_VOCAB;
}

size_t moe_verify_workspace_bytes(int32_t K, int32_t V) {
  return verify_shape_ok(K, V) ? verify_layout(K, V).total : 0;
}

moe_status moe_verify_accept(const float* logits, const float* draft_probs,
                             const int32_t* draft_tokens, const float* uniforms, int32_t K,
                             int32_t V, int32_t* out_tokens, int32_t* out_count, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!verify_shape_ok(K, V)) return MOE_ERR_INVALID;
  if (!logits || !out_tokens || !out_count || (K > 0 && !draft_tokens)) return MOE_ERR_INVALID;
  if (draft_probs && !uniforms) return MOE_ERR_INVALID;
  if (!aligned(logits, 4) || (draft_probs && !aligned(draft_probs, 4)) ||
      (uniforms && !aligned(uniforms, 4)) || !aligned(out_tokens, 4) || !aligned(out_count, 4) ||
      (draft_tokens && !aligned(draft_tokens, 4)))
    return MOE_ERR_INVALID;
  const VerifyLayout lay = verify_layout(K, V);
  const moe_status st = check_ws(ws, ws_bytes, lay.total);
  if (st != MOE_OK) return st;
  uint8_t* base = static_cast<uint8_t*>(ws);
  moe::VerifyArgs a{};
  a.L = logits;
  a.Q = draft_probs;
  a.d = draft_tokens;
  a.u = uniforms;
  a.out = out_tokens;
  a.count = out_count;
  a.st = reinterpret_cast<uint32_t*>(base + lay.st);
  a.cm = reinterpret_cast<float*>(base + lay.cm);
  a.ca = reinterpret_cast<int32_t*>(base + lay.ca);
  a.cs = reinterpret_cast<double*>(base + lay.cs);
  a.rowmz = reinterpret_cast<double*>(base + lay.rowmz);
  a.rmass = reinterpret_cast<double*>(base + lay.rmass);
  a.K = K;
  a.V = V;
  a.nch = moe::verify_chunks(V);
  const bool vec = V % 4 == 0 && aligned(logits, 16);
  return from_hip(moe::launch_verify(a, vec, stream));
}

moe_status moe_qk_norm_rope(uint16_t* qk, int32_t M, int32_t n_q_heads, int32_t n_k_heads,
                            int32_t head_dim, int64_t token_stride, const int32_t* positions,
                            const float* gamma_q, const float* gamma_k, float eps, float theta,
                            int32_t rot_dim, hipStream_t stream) {
  if (!qk || !positions || !gamma_q || !gamma_k) return MOE_ERR_INVALID;
  if (M < 1 || M > MOE_MAX_QK_TOKENS || n_q_heads < 0 || n_k_heads < 0) return MOE_ERR_INVALID;
  const int64_t nh = (int64_t)n_q_heads + n_k_heads;
  if (nh < 1 || nh > MOE_MAX_QK_HEADS) return MOE_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return MOE_ERR_INVALID;
  const int32_t per_lane = head_dim / 64;
  if (rot_dim < 0 || rot_dim > head_dim || rot_dim % (2 * per_lane)) return MOE_ERR_INVALID;
  if (token_stride < nh * head_dim || token_stride % 8) return MOE_ERR_INVALID;
  if (!(eps >= 0.0f) || !(theta > 0.0f) || !aligned(qk, 16) || !aligned(positions, 4) ||
      !aligned(gamma_q, 4) || !aligned(gamma_k, 4))
    return MOE_ERR_INVALID;
  moe::QkRopeArgs a{};
  a.qk = qk;
  a.pos = positions;
  a.gamma_q = gamma_q;
  a.gamma_k = gamma_k;
  a.eps = (double)eps;
  a.theta = (double)theta;
  a.stride = token_stride;
  a.M = M;
  a.nq = n_q_heads;
  a.nk = n_k_heads;
  a.hd = head_dim;
  a.rot = rot_dim;
  return from_hip(moe::launch_qk_norm_rope(a, stream));
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || !aligned(ws, 16)) return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_fill_zero(ws, ws_bytes, stream));
}

moe_status moe_quant_mx(int32_t wfmt, const float* w, int64_t rows, int64_t cols, void* q_out,
                        void* scale_out, int32_t* nonfinite_count, hipStream_t stream) {
  if (!w || !q_out || !scale_out) return MOE_ERR_INVALID;
  if (rows < 0 || cols < 0) return MOE_ERR_INVALID;
  if (!aligned(w, 16) || !aligned(q_out, 16)) return MOE_ERR_INVALID;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (wfmt == MOE_WFMT_MXFP4) {
    if (cols % 32) return MOE_ERR_INVALID;
    if (rows * (cols / 32) > ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    return from_hip(moe::launch_quant_mxfp4(w, rows, cols, static_cast<uint8_t*>(q_out),
                                            static_cast<uint8_t*>(scale_out), nonfinite_count,
                                            stream));
  }
  if (wfmt == MOE_WFMT_FP8_B128 || wfmt == MOE_WFMT_FP8_B128_A8) {
    if (cols % 16) return MOE_ERR_INVALID;
    if (!aligned(scale_out, 4)) return MOE_ERR_INVALID;
    if (((rows + 127) / 128) * ((cols + 127) / 128) > 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
    return from_hip(moe::launch_quant_fp8(w, rows, cols, static_cast<uint8_t*>(q_out),
                                          static_cast<float*>(scale_out), nonfinite_count,
                                          stream));
  }
  return MOE_ERR_INVALID;
}

moe_status moe_route_topk(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                          int32_t* topk_ids, float* topk_w, double* logits_out, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(layer);
  if (st != MOE_OK) return st;
  if (M < 1 || M > MOE_MAX_TOKENS) return MOE_ERR_INVALID;
  if (!x_bf16 || !topk_ids || !topk_w || !layer->router_w) return MOE_ERR_INVALID;
  if (!aligned(x_bf16, 16)) return MOE_ERR_INVALID;
  const WsLayout lay = layout(layer, M);
  st = check_ws(ws, ws_bytes, lay.total);
  if (st != MOE_OK) return st;
  uint8_t* base = static_cast<uint8_t*>(ws);
  moe::RouteArgs a{};
  a.x = x_bf16;
  a.wr = layer->router_w;
  a.bias = layer->router_b;
  a.logits = logits_out ? logits_out : reinterpret_cast<double*>(base + lay.logits);
  a.ids = topk_ids;
  a.w = topk_w;
  a.M = M;
  a.H = layer->hidden;
  a.E = layer->n_routed;
  a.k = layer->top_k;
  a.has_shared = layer->has_shared;
  return from_hip(moe::launch_route(a, stream));
}

}  // extern "C"

namespace {

// gate/up: the matrix-core form where it exists (several tokens), else the vector kernels.
hipError_t gate_up(const moe::FfnArgs& a, int wfmt, hipStream_t stream) {
  const hipError_t err = moe::launch_gate_up_mfma(a, wfmt, stream);
  return err == hipErrorNotSupported ? moe::launch_gate_up(a, wfmt, stream) : err;
}

// down + combine: the matrix-core form where it exists (several tokens), else the vector
// kernels.
hipError_t down_combine(const moe::FfnArgs& a, int wfmt, hipStream_t stream) {
  const hipError_t err = moe::launch_down_mfma(a, wfmt, stream);
  return err == hipErrorNotSupported ? moe::launch_down_combine(a, wfmt, stream) : err;
}

// Compute units of the current device, cached per device (0 when the query fails).
int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// Validation and argument setup shared by the FFN entry points; x and y may be null where the
// stage does not use them.
moe_status ffn_args(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                    const int32_t* topk_ids, const float* topk_w, uint16_t* y_bf16, void* ws,
                    size_t ws_bytes, int32_t* dev_status, moe::FfnArgs& a) {
  moe_status st = check_shape(layer);
  if (st != MOE_OK) return st;
  st = check_experts(layer);
  if (st != MOE_OK) return st;
  if (M < 1 || M > MOE_MAX_TOKENS) return MOE_ERR_INVALID;
  if (!topk_ids) return MOE_ERR_INVALID;
  if (x_bf16 && !aligned(x_bf16, 16)) return MOE_ERR_INVALID;
  const WsLayout lay = layout(layer, M);
  st = check_ws(ws, ws_bytes, lay.total);
  if (st != MOE_OK) return st;
  a = moe::FfnArgs{};
  a.w13 = static_cast<const uint8_t*>(layer->w13);
  a.w13s = layer->w13_scale;
  a.w2 = static_cast<const uint8_t*>(layer->w2);
  a.w2s = layer->w2_scale;
  a.x = x_bf16;
  a.ids = topk_ids;
  a.topk_w = topk_w;
  a.a_buf = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + lay.a_buf);
  a.o_buf = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + lay.o_buf);
  a.y = y_bf16;
  a.status = dev_status;
  a.M = M;
  a.S = layer->top_k + layer->has_shared;
  a.H = layer->hidden;
  a.I = layer->inter;
  a.n_experts = layer->n_routed + layer->has_shared;
  a.has_shared = layer->has_shared;
  a.cus = device_cus();
  uint8_t* base = static_cast<uint8_t*>(ws);
  a.xq = reinterpret_cast<uint16_t*>(base + lay.xq);
  a.x_scales = reinterpret_cast<float*>(base + lay.x_scales);
  a.aq = reinterpret_cast<float*>(base + lay.aq);
  a.a_scales = reinterpret_cast<float*>(base + lay.a_scales);
  return MOE_OK;
}

// Route, gate/up, down and combine of one layer: the logits launch, then the gate/up kernel
// selects the experts itself (the router's rule, bit-identical ids and weights to the top-k
// launch it replaces) and publishes them for the down and combine launches.  With one_launch
// (one token only) the whole layer in one launch (hipErrorNotSupported, nothing enqueued, for
// shapes it is not built for).  fa's ids / topk_w must be ra's outputs.
hipError_t layer_launch(const moe_layer& L, const moe::RouteArgs& ra, const moe::FfnArgs& fa,
                        uint8_t* ws, const WsLayout& lay, bool one_launch, hipStream_t stream) {
  moe::FfnArgs g = fa;
  g.ids = nullptr;
  g.logits = ra.logits;
  g.ids_out = ra.ids;
  g.w_out = ra.w;
  g.E_routed = L.n_routed;
  g.k_routed = L.top_k;
  if (one_launch) {
    if (fa.M != 1) return hipErrorNotSupported;
    moe::FfnArgs f = g;
    f.a_buf = reinterpret_cast<float*>(ws + lay.a64);
    f.o_buf = reinterpret_cast<float*>(ws + lay.o64);
    return moe::launch_layer_m1(f, ra, L.wfmt, reinterpret_cast<uint32_t*>(ws + lay.counters),
                                stream);
  }
  hipError_t err = moe::launch_logits_only(ra, stream);
  if (err == hipSuccess) err = gate_up(g, L.wfmt, stream);
  if (err == hipSuccess) err = down_combine(fa, L.wfmt, stream);
  return err;
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn_decode(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                                 const int32_t* topk_ids, const float* topk_w, uint16_t* y_bf16,
                                 void* ws, size_t ws_bytes, int32_t* dev_status,
                                 hipStream_t stream) {
  if (!x_bf16 || !topk_w || !y_bf16) return MOE_ERR_INVALID;
  moe::FfnArgs a;
  const moe_status st =
      ffn_args(layer, x_bf16, M, topk_ids, topk_w, y_bf16, ws, ws_bytes, dev_status, a);
  if (st != MOE_OK) return st;
  hipError_t err = gate_up(a, layer->wfmt, stream);
  if (err == hipSuccess) err = down_combine(a, layer->wfmt, stream);
  return from_hip(err);
}

moe_status moe_expert_gate_up(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                              const int32_t* topk_ids, void* ws, size_t ws_bytes,
                              int32_t* dev_status, hipStream_t stream) {
  if (!x_bf16) return MOE_ERR_INVALID;
  moe::FfnArgs a;
  const moe_status st =
      ffn_args(layer, x_bf16, M, topk_ids, nullptr, nullptr, ws, ws_bytes, dev_status, a);
  if (st != MOE_OK) return st;
  return from_hip(gate_up(a, layer->wfmt, stream));
}

moe_status moe_expert_down_combine(const moe_layer* layer, int32_t M, const int32_t* topk_ids,
                                   const float* topk_w, uint16_t* y_bf16, void* ws,
                                   size_t ws_bytes, int32_t* dev_status, hipStream_t stream) {
  if (!topk_w || !y_bf16) return MOE_ERR_INVALID;
  moe::FfnArgs a;
  const moe_status st =
      ffn_args(layer, nullptr, M, topk_ids, topk_w, y_bf16, ws, ws_bytes, dev_status, a);
  if (st != MOE_OK) return st;
  return from_hip(down_combine(a, layer->wfmt, stream));
}

moe_status moe_layer_decode(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                            int32_t* topk_ids, float* topk_w, double* logits_out,
                            uint16_t* y_bf16, void* ws, size_t ws_bytes, int32_t* dev_status,
                            hipStream_t stream) {
  return layer_decode_impl(layer, x_bf16, M, topk_ids, topk_w, logits_out, y_bf16, ws, ws_bytes,
                           dev_status, false, stream);
}

moe_status moe_layer_decode_one_launch(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                                       int32_t* topk_ids, float* topk_w, double* logits_out,
                                       uint16_t* y_bf16, void* ws, size_t ws_bytes,
                                       int32_t* dev_status, hipStream_t stream) {
  if (M != 1) return MOE_ERR_UNSUPPORTED;
  return layer_decode_impl(layer, x_bf16, M, topk_ids, topk_w, logits_out, y_bf16, ws, ws_bytes,
                           dev_status, true, stream);
}

moe_status moe_layer_decode_static(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                                   int32_t* topk_ids, float* topk_w, double* logits_out,
                                   uint16_t* y_bf16, int32_t* dev_status, hipStream_t stream) {
  const moe_status st = check_shape(layer);
  if (st != MOE_OK) return st;
  if (M < 1 || M > MOE_MAX_TOKENS) return MOE_ERR_INVALID;
  if (layout(layer, M).total > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const moe_status sst = static_scratch(stream, &ws);
  if (sst != MOE_OK) return sst;
  return layer_decode_impl(layer, x_bf16, M, topk_ids, topk_w, logits_out, y_bf16, ws,
                           MOE_STATIC_SCRATCH_BYTES, dev_status, false, stream);
}

}  // extern "C"

namespace {

moe_status layer_decode_impl(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                             int32_t* topk_ids, float* topk_w, double* logits_out,
                             uint16_t* y_bf16, void* ws, size_t ws_bytes, int32_t* dev_status,
                             bool one_launch, hipStream_t stream) {
  moe_status st = check_shape(layer);
  if (st != MOE_OK) return st;
  if (!x_bf16 || !topk_ids || !topk_w || !y_bf16 || !layer->router_w) return MOE_ERR_INVALID;
  moe::FfnArgs fa;
  st = ffn_args(layer, x_bf16, M, topk_ids, topk_w, y_bf16, ws, ws_bytes, dev_status, fa);
  if (st != MOE_OK) return st;
  const WsLayout lay = layout(layer, M);
  moe::RouteArgs ra{};
  ra.x = x_bf16;
  ra.wr = layer->router_w;
  ra.bias = layer->router_b;
  ra.logits = logits_out ? logits_out
                         : reinterpret_cast<double*>(static_cast<uint8_t*>(ws) + lay.logits);
  ra.ids = topk_ids;
  ra.w = topk_w;
  ra.M = M;
  ra.H = layer->hidden;
  ra.E = layer->n_routed;
  ra.k = layer->top_k;
  ra.has_shared = layer->has_shared;
  const hipError_t err =
      layer_launch(*layer, ra, fa, static_cast<uint8_t*>(ws), lay, one_launch, stream);
  return err == hipErrorNotSupported ? MOE_ERR_UNSUPPORTED : from_hip(err);
}

}  // namespace

extern "C" {

moe_status moe_layer_stack_persistent(const moe_layer* layers, int32_t n_layers, float rms_eps,
                                      uint16_t* h_bf16, int32_t M, void* ws, size_t ws_bytes,
                                      void* trace, hipStream_t stream) {
  if (!layers || n_layers < 1 || !h_bf16) return MOE_ERR_INVALID;
  if (M < 1 || M > MOE_MAX_TOKENS) return MOE_ERR_INVALID;
  if (!(rms_eps >= 0.0f) || !aligned(h_bf16, 16)) return MOE_ERR_INVALID;
  const moe_layer& L0 = layers[0];
  for (int32_t l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    moe_status st = check_shape(&L);
    if (st != MOE_OK) return st;
    st = check_experts(&L);
    if (st != MOE_OK) return st;
    if (L.wfmt != L0.wfmt || L.hidden != L0.hidden || L.inter != L0.inter ||
        L.n_routed != L0.n_routed || L.top_k != L0.top_k || L.has_shared != L0.has_shared)
      return MOE_ERR_INVALID;
    if (!L.router_w || !L.rms_gamma || !aligned(L.rms_gamma, 16)) return MOE_ERR_INVALID;
  }
  const WsLayout lay = layout(&L0, M);
  const moe_status wst = check_ws(ws, ws_bytes, lay.total);
  if (wst != MOE_OK) return wst;
  if (trace && !aligned(trace, 16)) return MOE_ERR_INVALID;
  uint8_t* base = static_cast<uint8_t*>(ws);
  const int32_t H = L0.hidden, S = L0.top_k + L0.has_shared;
  const size_t rec = (size_t)M * H * sizeof(uint16_t) + 2 * (size_t)M * S * sizeof(int32_t);
  uint16_t* xn = reinterpret_cast<uint16_t*>(base + lay.xn);
  for (int32_t l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    uint8_t* r = trace ? static_cast<uint8_t*>(trace) + l * rec : nullptr;
    int32_t* ids = r ? reinterpret_cast<int32_t*>(r + (size_t)M * H * sizeof(uint16_t))
                     : reinterpret_cast<int32_t*>(base + lay.ids);
    float* w = r ? reinterpret_cast<float*>(r + (size_t)M * H * sizeof(uint16_t) +
                                            (size_t)M * S * sizeof(int32_t))
                 : reinterpret_cast<float*>(base + lay.w);
    moe::RouteArgs ra{};
    ra.x = h_bf16;
    ra.wr = L.router_w;
    ra.bias = L.router_b;
    ra.logits = reinterpret_cast<double*>(base + lay.logits);
    ra.ids = ids;
    ra.w = w;
    ra.gamma = L.rms_gamma;
    ra.eps = (double)rms_eps;
    ra.xn_out = xn;
    ra.x_copy = r ? reinterpret_cast<uint16_t*>(r) : nullptr;
    ra.M = M;
    ra.H = H;
    ra.E = L.n_routed;
    ra.k = L.top_k;
    ra.has_shared = L.has_shared;
    hipError_t err = moe::launch_rmsnorm(ra, stream);  // h -> xn (and h into the trace)
    if (err != hipSuccess) return MOE_ERR_HIP;
    ra.x = xn;  // the router and the experts see the normalized activations
    moe::FfnArgs fa;
    const moe_status st = ffn_args(&L, xn, M, ids, w, h_bf16, ws, ws_bytes, nullptr, fa);
    if (st != MOE_OK) return st;
    fa.residual = true;
    err = layer_launch(L, ra, fa, base, lay, false, stream);
    if (err != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // extern "C"
