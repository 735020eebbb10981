/* Plain CPU reference ("oracle") of the MoE decode layer.  TEST
 * INFRASTRUCTURE ONLY: nothing but the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the GPU library never does.
 *
 * It shares no code with the GPU library.  All arithmetic is fp64 unless a
 * step fixes another precision; every function states the passage of the
 * pages it follows (see moe_oracle.c). */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_WFMT_MXFP4 = 1, ORC_WFMT_FP8_B128 = 2, ORC_WFMT_FP8_B128_A8 = 3 };

/* One MoE layer's packed experts.  Expert e's matrices are
 *   W13_e [2I][H] (gate rows [0,I), up rows [I,2I)) and W2_e [H][I];
 * each is row-major with K (the reduction axis) contiguous:
 *   MXFP4   : codes u8 [rows][K/2] (low nibble = even element), scales u8 E8M0 [rows][K/32]
 *   FP8_B128: codes u8 E4M3FN [rows][K],  scales fp32 [rows/128][K/128]
 *   FP8_B128_A8: the FP8_B128 weights; the FFN also quantizes its activations (W8A8)
 * Pointers may be NULL for experts that no token references. */
typedef struct {
  int32_t wfmt, hidden, inter, n_experts;
  const uint8_t* const* w13_q;
  const void* const* w13_s;
  const uint8_t* const* w2_q;
  const void* const* w2_s;
} orc_experts;

void orc_set_threads(int32_t n);
int32_t orc_get_threads(void);

double orc_e2m1_value(uint32_t code);
double orc_e8m0_value(uint32_t code);
double orc_e4m3_value(uint32_t code);
uint32_t orc_e2m1_rne(double t);   /* |t| -> 3-bit magnitude code, saturating */
uint32_t orc_e4m3_rne(double t);   /* |t| -> 7-bit magnitude code, saturating */
uint16_t orc_bf16_from_double(double d);

/* Quantizers.  Return the number of non-finite inputs seen. */
int64_t orc_quant_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s);
int64_t orc_quant_fp8_b128(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s);
/* Live activation quantizer of the W8A8 variant: v fp32 [n] (n % 128 == 0) -> codes u8 [n],
 * scales fp32 [n/128].  Returns the number of non-finite inputs seen. */
int64_t orc_quant_act_fp8(const float* v, int64_t n, uint8_t* q, float* s);
void orc_dequant(int32_t wfmt, const uint8_t* q, const void* s, int64_t rows, int64_t cols,
                 double* out);

/* Router: x bf16 [M][H], wr fp32 [E][H], b fp32 [E] or NULL.
 * ids int32 [M][S], w fp64 [M][S] with S = k + has_shared; logits fp64 [M][E];
 * gap fp64 [M] = (k-th largest logit) - ((k+1)-th largest), +inf when k == E. */
void orc_route(const uint16_t* x, int32_t M, int32_t H, const float* wr, const float* b,
               int32_t E, int32_t k, int32_t has_shared, int32_t* ids, double* w,
               double* logits, double* gap);

/* Expert FFN + combine: y fp64 [M][H].  token_mask (nullable) selects tokens;
 * rows of unselected tokens are set to NaN. */
void orc_expert_ffn(const orc_experts* L, const uint16_t* x, int32_t M, const int32_t* ids,
                    const float* w, int32_t S, const uint8_t* token_mask, double* y);

/* RMSNorm to bf16: out = bf16((h * r) * gamma), r = 1/sqrt(mean(h^2) + eps). */
void orc_rmsnorm(const uint16_t* h, int32_t M, int32_t H, const float* gamma, double eps,
                 uint16_t* out);
/* Residual: out = bf16(h + y). */
void orc_residual(const uint16_t* h, const double* y, int64_t n, uint16_t* out);

/* Verify-acceptance of one speculative block: L fp32 [K+1][V] target logits, Q fp32 [K][V]
 * draft probabilities (NULL: greedy), d int32 [K] draft tokens, u fp32 [K+1] uniforms in [0,1)
 * (unused when greedy).  out int32 [K+1]; returns the number of tokens written (n + 1).
 * margin (nullable, [2]): smallest relative distance to its threshold of an accept test, then
 * of the draw. */
int32_t orc_verify(const float* L, const float* Q, const int32_t* d, const float* u, int32_t K,
                   int32_t V, int32_t* out, double* margin);

/* Fused QK-norm + RoPE of M tokens: x bf16 heads (token t at x + t*stride, head h at h*hd;
 * q heads [0, nq) with gamma_q, k heads [nq, nh) with gamma_k), pos int32 [M].
 * y_f64 (nullable) / y_bf16: [M][nh][hd], unrounded / rounded once. */
void orc_qk_norm_rope(const uint16_t* x, int32_t M, int32_t nq, int32_t nh, int32_t hd,
                      int64_t stride, const int32_t* pos, const float* gq, const float* gk,
                      double eps, double theta, int32_t rot, double* y_f64, uint16_t* y_bf16);

#ifdef __cplusplus
}
#endif
#endif
