/* moe_mx -- MoE decode layer for AMD MI355X (gfx950): C ABI.
 *
 * The step these calls implement is the batch-1 / few-token (M = 1..16) decode
 * step of a sparse MoE layer, which is bound by reading the selected experts'
 * weights from HBM:
 *   - top-k routing with the shared expert fused as the last slot
 *     (blogs.novita.ai, "Optimizing GLM4-MoE for production", section 1, shared
 *     experts fusion: top 9 of 161, the shared expert always ninth);
 *   - per selected expert a SwiGLU FFN on low-precision weights: MXFP4 (E2M1
 *     codes, one E8M0 exponent per 32 values along K) or FP8 E4M3 with fp32
 *     scales per 128x128 block (molayo1419.me, "Xiaomi가 어떻게 1조 개의 파라미터를
 *     가진 모델에서 초당 1,000 토큰을 달성했는가", section 2, expert-only MXFP4);
 *   - the weighted combine of the slots;
 *   - an optional stack of layers, RMSNorm -> router -> experts -> residual,
 *     in one call that enqueues every layer's kernels back to back, graph-
 *     capturable, with no host synchronization (same page, section 1 on the
 *     execution gap between operators and the persistent engine it names).
 *
 * Conventions for every call:
 *   - Data pointers are DEVICE memory owned by the caller unless stated.  The
 *     library allocates no device memory, keeps no state between calls (apart
 *     from the static scratch of moe_layer_decode_static), and never
 *     synchronizes the host: every call only enqueues work on `stream`.
 *   - Descriptors (moe_layer) are read on the host during the call and may be
 *     freed on return.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns an error and enqueues nothing.  A failed launch
 *     returns MOE_ERR_HIP.  No C++ exception crosses this interface.
 *   - bf16 values travel as raw uint16 bit patterns.
 *   - Calls that take a workspace need `ws` of at least moe_workspace_bytes()
 *     bytes, 256-byte aligned, zero-filled once after allocation (for example
 *     with moe_workspace_init).  Every call leaves the workspace's counters at
 *     zero again, so one workspace serves any sequence of calls on one stream;
 *     calls that overlap in time (other streams) need their own workspace.
 *
 * Packed expert tensors (all experts of a layer contiguous, the shared expert
 * stored last at index n_routed; K, the reduction axis, contiguous):
 *   W13 [E+1][2I][H]: rows [0,I) gate, rows [I,2I) up;   W2 [E+1][H][I].
 *   MXFP4    codes  u8 [rows][K/2]  (element 2j in the low nibble, 2j+1 high)
 *            scales u8 [rows][K/32] (E8M0: 2^(s-127); 255 = NaN)
 *   FP8_B128 codes  u8 [rows][K]    (OCP E4M3FN; FP8_B128_A8 likewise)
 *            scales fp32 [ceil(rows/128)][ceil(K/128)] per expert matrix (the last
 *            block along a side that is not a multiple of 128 is partial)
 * Codes and scales must be 16-byte aligned.
 */
#ifndef MOE_MX_H
#define MOE_MX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* null pointer, misalignment or a shape outside the limits */
  MOE_ERR_UNSUPPORTED = 2, /* well-formed but not supported by this library */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} moe_status;

/* FP8_B128_A8 (W8A8): the FP8_B128 weights (same layout and quantizer); the expert FFN also
 * quantizes its activations live, inside the weight-streaming kernels (Sionic
 * "glm-5-2-b300-kernel-mtp-serving", table under "what it solves" and idea 1: live FP8
 * activation quantization fused into the expert GEMM; idea 3: it changes the outputs, so its
 * fidelity cost is measured).  Per 128 consecutive values along K of one token's input x and of
 * its SwiGLU output a (fp32): s = fp32(amax/448), 1 for an all-zero block, NaN for a block
 * holding a non-finite value; the value used is s times the E4M3 value nearest fp32(v/s), ties
 * to even, saturating at 448.  One token (the batch-1 step the pages measure) is quantized
 * inside the weight-streaming kernels; several tokens (a verify block) by two small passes into
 * the workspace. */
typedef enum {
  MOE_WFMT_MXFP4 = 1,
  MOE_WFMT_FP8_B128 = 2,
  MOE_WFMT_FP8_B128_A8 = 3
} moe_wfmt;

/* Limits checked by every call. */
#define MOE_MAX_TOKENS 16  /* M: decode token or speculative-verify block */
#define MOE_MAX_SLOTS 16   /* k + has_shared */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_VOCAB (1 << 24) /* V of moe_verify_accept */
#define MOE_MAX_QK_TOKENS 65536 /* M of moe_qk_norm_rope */
#define MOE_MAX_QK_HEADS 1024

/* One MoE layer (device pointers; the struct itself is host memory). */
typedef struct {
  int32_t wfmt;        /* moe_wfmt */
  int32_t hidden;      /* H: multiple of 128 */
  int32_t inter;       /* I: multiple of 32; FP8_B128_A8 (W8A8): multiple of 128 */
  int32_t n_routed;    /* E routed experts */
  int32_t top_k;       /* k routed experts per token, 1 <= k <= E */
  int32_t has_shared;  /* 1: a shared expert is stored at index E and fused as slot k */
  const void* w13;     /* packed codes of W13, layout above */
  const void* w13_scale;
  const void* w2;      /* packed codes of W2 */
  const void* w2_scale;
  const float* router_w; /* [E][H] fp32 */
  const float* router_b; /* [E] fp32 or NULL: added to the logit before ranking and sigmoid */
  const float* rms_gamma; /* [H] fp32: RMSNorm gain, used by the layer stack only */
} moe_layer;

/* Quantize fp32 weights w [rows][cols] (cols = K contiguous) into the packed format.
 *   MXFP4: shared exponent X = floor(log2(amax)) - 2 per 32-element block along K, clamped to
 *     [-127, 127] (all-zero block: X = -127); code = sign | nearest-even E2M1 of |v|/2^X,
 *     saturating at 6; cols % 32 == 0.  (molayo, Xiaomi 1T page, section 2, MXFP4 with QAT:
 *     32-value blocks under one exponent as the MX specification defines.)
 *   FP8_B128, FP8_B128_A8: per 128x128 block s = fp32(amax/448) (1 for an all-zero block),
 *     code = sign | nearest-even E4M3FN of fp32(v/s), saturating at 448; cols % 16 == 0.
 *     Blocks tile the matrix from its origin; along a side that is not a multiple of 128 the
 *     last block covers the remaining rows / columns (one tensor-parallel rank's slice of the
 *     GLM-4.7 intermediate, 1536 / 8 = 192: blogs.novita.ai, "Optimizing GLM4-MoE for
 *     production", section 1).
 * q_out: codes (MXFP4 rows*cols/2 bytes, FP8 rows*cols bytes); scale_out: MXFP4 u8
 * [rows][cols/32], FP8 fp32 [ceil(rows/128)][ceil(cols/128)].  A block holding a non-finite
 * input gets a NaN scale (0xFF / fp32 NaN) and zero (MXFP4) or NaN (FP8) codes, and the number
 * of non-finite inputs is added atomically to *nonfinite_count (device int32, nullable, not
 * cleared by the call).  Bit-exact with the reference quantizer. */
moe_status moe_quant_mx(int32_t wfmt, const float* w, int64_t rows, int64_t cols, void* q_out,
                        void* scale_out, int32_t* nonfinite_count, hipStream_t stream);

/* Router for M tokens x bf16 [M][H] (novita page section 1; molayo page section 1, sparse
 * top-k routing): logit l_e = x . Wr_e (+ b_e) accumulated in fp64; experts ranked by
 * (logit descending, index ascending); the k best get w = sigmoid(l)/sum of the k sigmoids;
 * with has_shared, slot k holds id E with weight 1.0.
 * Outputs: topk_ids int32 [M][S], topk_w fp32 [M][S] (S = k + has_shared);
 * logits_out fp64 [M][E] (nullable).  Needs the workspace. */
moe_status moe_route_topk(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                          int32_t* topk_ids, float* topk_w, double* logits_out, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Expert FFN and combine for M tokens: for every token t and slot j with e = ids[t][j],
 * o = W2_e (silu(Wg_e x_t) * (Wu_e x_t)), silu(z) = z * sigmoid(z); y_t = sum_j w[t][j] o,
 * fp32 accumulation, y rounded to bf16 (nearest even).  Each distinct expert's weights are
 * read once per call however many tokens select it (molayo page section 1, decode is bound by
 * reading active weights; Sionic "glm-5-2-b300-kernel-mtp-serving", idea 3: one weight stream
 * serves a whole verify block).  Ids outside [0, E + has_shared) contribute nothing and set
 * bit 0 of *dev_status (device int32, nullable, not cleared by the call).
 * y_bf16 [M][H]; topk_ids/topk_w as produced by moe_route_topk. */
moe_status moe_expert_ffn_decode(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                                 const int32_t* topk_ids, const float* topk_w, uint16_t* y_bf16,
                                 void* ws, size_t ws_bytes, int32_t* dev_status,
                                 hipStream_t stream);

/* The two weight-streaming stages of moe_expert_ffn_decode as separate calls; the pair, in this
 * order on one stream with one workspace, gives the same bits as moe_expert_ffn_decode.
 * moe_expert_gate_up: a = silu(Wg_e x_t) * (Wu_e x_t) for every (token, slot) pair, fp32, into
 *   the workspace (reads every active expert's W13 once).
 * moe_expert_down_combine: y_t = sum_j w[t][j] W2_e a_(t,j) in slot order, bf16 (reads every
 *   active expert's W2 once); needs the workspace written by moe_expert_gate_up for the same
 *   layer, M and ids.
 * Arguments, errors and dev_status as for moe_expert_ffn_decode. */
moe_status moe_expert_gate_up(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                              const int32_t* topk_ids, void* ws, size_t ws_bytes,
                              int32_t* dev_status, hipStream_t stream);
moe_status moe_expert_down_combine(const moe_layer* layer, int32_t M, const int32_t* topk_ids,
                                   const float* topk_w, uint16_t* y_bf16, void* ws,
                                   size_t ws_bytes, int32_t* dev_status, hipStream_t stream);

/* Route + expert FFN + combine of one layer: the same results, bit for bit, as
 * moe_route_topk followed by moe_expert_ffn_decode on the same stream (ids, weights, logits
 * when logits_out is set, y).  With one token (M = 1) the gate/up kernel selects the experts
 * from the logits itself, by the router's rule, instead of waiting for a separate top-k launch
 * (molayo page section 1: at high token rates the operator boundaries dominate), and publishes
 * ids and weights for the kernels that follow: four launches instead of five.  Arguments,
 * errors and dev_status as for the two calls; the workspace of moe_workspace_bytes. */
moe_status moe_layer_decode(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                            int32_t* topk_ids, float* topk_w, double* logits_out,
                            uint16_t* y_bf16, void* ws, size_t ws_bytes, int32_t* dev_status,
                            hipStream_t stream);

/* moe_layer_decode for one token (M = 1) as ONE kernel launch: the router's logits, the
 * selection, gate/up + SwiGLU, down and the combine run in a single resident grid (molayo page,
 * section 1: the page's engine removes the gaps between operators with one persistent kernel;
 * novita page, section 1: the shared expert, fused as the last slot, needs no routing, so its
 * gate/up streams while the logits are computed).  Waves hand the logits, the SwiGLU outputs and
 * the slot outputs to each other through the workspace, each value carrying the call's epoch;
 * there are no atomics, fences or grid-wide barriers.  Same arguments, results (bit for bit)
 * and workspace as moe_layer_decode.  Built for hidden 5120 (FP8_B128: intermediate 1536 or 192;
 * MXFP4: 1536 or 192) and hidden 7168 (MXFP4: 2048 or 256); other shapes and M > 1 return
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  Bit 1 of *dev_status is set if a hand-off
 * wait gave up (it cannot while the whole grid is resident; the call then returns garbage
 * rather than hang).  Measured slower than moe_layer_decode's chain of launches on MI355X (the
 * waits for each expert's slowest producer cost more than the kernel boundaries they replace),
 * so moe_layer_decode keeps the chain. */
moe_status moe_layer_decode_one_launch(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                                       int32_t* topk_ids, float* topk_w, double* logits_out,
                                       uint16_t* y_bf16, void* ws, size_t ws_bytes,
                                       int32_t* dev_status, hipStream_t stream);

/* moe_layer_decode for callers that cannot allocate device memory or own a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus the workspace), results, launches and errors as moe_layer_decode; the
 * workspace is a library-owned scratch array of MOE_STATIC_SCRATCH_BYTES bytes on each GPU it
 * runs on, held until the process ends.  The call allocates nothing (no hipMalloc or hipFree,
 * no allocating library routine).  Shapes whose workspace (moe_workspace_bytes) exceeds
 * MOE_STATIC_SCRATCH_BYTES return MOE_ERR_UNSUPPORTED before anything is enqueued.  Every call
 * on one GPU shares that GPU's scratch, which keeps the last call's contents: calls that
 * overlap in time on one GPU (several streams or host threads) race and must be serialized by
 * the caller.  The first call on a GPU also enqueues, on `stream`, one fill kernel that clears
 * the scratch's counter area. */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)
moe_status moe_layer_decode_static(const moe_layer* layer, const uint16_t* x_bf16, int32_t M,
                                   int32_t* topk_ids, float* topk_w, double* logits_out,
                                   uint16_t* y_bf16, int32_t* dev_status, hipStream_t stream);

/* n_layers consecutive pre-norm residual layers applied to h [M][H] bf16 in place
 * (molayo page, section 1: the decode step runs layer after layer, each reading its active
 * experts; the layers are enqueued back to back on the stream with no host synchronization, so
 * the whole stack is one graph-capturable call):
 *   xn = bf16((h * r) * gamma), r = 1/sqrt(mean(h^2) + eps) in fp64, each element rounded once;
 *   ids, w = route(xn);  y = experts(xn, ids, w) in fp32;  h = bf16(h + y), rounded once.
 * All layers share wfmt, hidden, inter, n_routed, top_k and has_shared, and need router_w and
 * rms_gamma (16-byte aligned); otherwise MOE_ERR_INVALID.  rms_eps >= 0.
 * trace (nullable, 16-byte aligned): per layer l a record of M*H*2 + 8*M*S bytes at offset
 * l * (M*H*2 + 8*M*S): the layer's input h (bf16 [M][H]), then ids (int32 [M][S]), then
 * w (fp32 [M][S]).  Needs the workspace of moe_workspace_bytes(layers, n_layers, M). */
moe_status moe_layer_stack_persistent(const moe_layer* layers, int32_t n_layers, float rms_eps,
                                      uint16_t* h_bf16, int32_t M, void* ws, size_t ws_bytes,
                                      void* trace, hipStream_t stream);

/* Verify-acceptance of one speculative block: the step after the backbone's verify forward
 * over K draft tokens (molayo page section 3: a draft proposes K tokens, the backbone scores
 * them in one forward, and rejection sampling accepts a prefix without changing the output
 * distribution; Sionic "glm-5-2-b300-kernel-mtp-serving", idea 3: the leading draft tokens that
 * agree with the main model are confirmed at once).  The pages give no formulas; this is the
 * standard speculative-sampling rule:
 *   Row i of logits (fp32 [K+1][V], finite or -inf, one finite value per row at least) scores
 *   the token after the prefix and the first i draft tokens; p_i = softmax(row i).  The bulk
 *   exponentials are fp32 summed in fp64, the accept test's own exponential fp64, so a decision
 *   can differ from exact arithmetic only within about 1e-6 of its threshold.
 *   Greedy (draft_probs NULL): draft_tokens[i] is accepted while it equals argmax of row i
 *     (lowest index on ties); the next token is the argmax of the first row not matched (row K
 *     when all are).
 *   Sampling (draft_probs fp32 [K][V], the draft's distribution at each position; uniforms fp32
 *     [K+1] in [0, 1), drawn by the caller): draft token i is accepted iff
 *     uniforms[i] * q_i(d_i) < p_i(d_i).  At the first rejection j the next token is drawn from
 *     max(0, p_j - q_j) (from p_j if that is zero everywhere); after a full accept from p_K.  A
 *     draw takes the smallest index whose prefix sum in index order exceeds uniforms[K] times
 *     the total.
 *   A draft token outside [0, V) is never accepted.
 * Outputs (device): out_tokens int32 [K+1] receives the n accepted draft tokens then the next
 * token; *out_count = n + 1 (int32).  Entries past n are left unchanged.
 * 0 <= K < MOE_MAX_TOKENS, 1 <= V <= MOE_MAX_VOCAB, pointers 4-byte aligned (logits 16-byte
 * aligned with V % 4 == 0 take the vector path).  Needs a workspace of
 * moe_verify_workspace_bytes(K, V) bytes, 256-byte aligned; it holds no state between calls,
 * and calls that overlap in time need their own.  Four launches with draft_probs, two without;
 * no host synchronization. */
moe_status moe_verify_accept(const float* logits, const float* draft_probs,
                             const int32_t* draft_tokens, const float* uniforms, int32_t K,
                             int32_t V, int32_t* out_tokens, int32_t* out_count, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of moe_verify_accept for K draft tokens over a vocabulary of V; 0 when the
 * shape is outside the limits. */
size_t moe_verify_workspace_bytes(int32_t K, int32_t V);

/* Fused QK-norm + RoPE, in place: the attention-side pre-norms of a step in one kernel
 * (Novita "Optimizing GLM4-MoE for production", section 2: the head-wise RMSNorm of Q and K and
 * the rotary embedding are both per-head work and fuse into one kernel; in the GLM4-MoE variant
 * only half of each head rotates.  molayo page, section 1: RMSNorm and RoPE are among the
 * operators whose boundaries cost time at high token rates).
 * qk: bf16 device buffer; token t's heads start at qk + t * token_stride (elements): n_q_heads
 * query heads then n_k_heads key heads, head_dim contiguous values each (other data, such as V,
 * may follow within the stride and is not touched).  For token t and head h with x its values:
 *   r = 1/sqrt(sum(x^2)/head_dim + eps);  n_k = (x_k * r) * gamma_k  (gamma_q for query heads);
 *   the first rot_dim values rotate in pairs (i, i + rot_dim/2), i < rot_dim/2, by the angle
 *   positions[t] * theta^(-2i/rot_dim):  y_i = n_i c - n_j s,  y_j = n_j c + n_i s;
 *   the rest keep n.  fp64 throughout, each value rounded once to bf16 (nearest even).
 * positions int32 [M]; gamma_q, gamma_k fp32 [head_dim].  head_dim 64, 128 or 256; rot_dim in
 * [0, head_dim] a multiple of head_dim/32; token_stride >= (n_q_heads + n_k_heads) * head_dim
 * and a multiple of 8; qk 16-byte aligned; eps >= 0, theta > 0; 1 <= M <= MOE_MAX_QK_TOKENS,
 * 1 <= n_q_heads + n_k_heads <= MOE_MAX_QK_HEADS.  One launch, no workspace. */
moe_status moe_qk_norm_rope(uint16_t* qk, int32_t M, int32_t n_q_heads, int32_t n_k_heads,
                            int32_t head_dim, int64_t token_stride, const int32_t* positions,
                            const float* gamma_q, const float* gamma_k, float eps, float theta,
                            int32_t rot_dim, hipStream_t stream);

/* Workspace bytes that every call above needs for these layers and up to M tokens. */
size_t moe_workspace_bytes(const moe_layer* layers, int32_t n_layers, int32_t M);

/* Zero-fill a workspace (a fill kernel, safe under stream capture). */
moe_status moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Static string naming a status. */
const char* moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MX_H */
