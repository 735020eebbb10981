/* Plain CPU reference of the MoE decode layer -- TEST INFRASTRUCTURE ONLY.
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code with the GPU library.
 *
 * Pages cited (titles as printed; Korean pages):
 *   [XIAOMI] molayo1419.me, "Xiaomi가 어떻게 1조 개의 파라미터를 가진 모델에서 초당
 *            1,000 토큰을 달성했는가: LLM 추론 최적화 심층 분석"
 *   [SIONIC] d9249.github.io, "glm-5-2-b300-kernel-mtp-serving" (Sionic GLM-5.2 on B300)
 *   [NOVITA] blogs.novita.ai, "Optimizing GLM4-MoE for production"
 *
 * Where the pages are silent the code says which reading it takes.  All
 * arithmetic is fp64 unless a step fixes another precision.  The loops are
 * written in the order of the definitions; OpenMP only splits independent
 * outputs across threads and never changes any sum's order. */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static int g_threads = 1;

void orc_set_threads(int32_t n) { g_threads = n < 1 ? 1 : n; }
int32_t orc_get_threads(void) { return g_threads; }

/* ---- element formats ----------------------------------------------------------------------
 * [XIAOMI] §2, "QAT를 적용한 MXFP4": experts use MXFP4, blocks of 32 values that share one
 * exponent as the MX specification defines, and an FP4 element has only 16 distinct codes
 * (§2, "수치로 보는 대역폭 병목 현상").  The pages print no bit layout, so the element is
 * read as the MX specification's E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 * mantissa; exponent 0 is subnormal.  (The page's "3-bit mantissa" is read as the three
 * bits besides the sign.) */
double orc_e2m1_value(uint32_t code) {
  const uint32_t sign = (code >> 3) & 1u, exp = (code >> 1) & 3u, man = code & 1u;
  double mag;
  if (exp == 0)
    mag = ldexp((double)man / 2.0, 1 - 1);            /* subnormal: 2^(1-bias) * m/2 */
  else
    mag = ldexp(1.0 + (double)man / 2.0, (int)exp - 1); /* normal: 2^(e-bias) * (1+m/2) */
  return sign ? -mag : mag;
}

/* The shared block scale: E8M0, value 2^(code-127); code 255 is NaN (MX specification). */
double orc_e8m0_value(uint32_t code) {
  code &= 0xFFu;
  if (code == 0xFFu) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* FP8 E4M3 (OCP "FN" variant: no infinities, only S.1111.111 is NaN, max 448): bit 7 sign,
 * bits 6..3 exponent (bias 7), bits 2..0 mantissa.  The FP8 expert baseline is named in
 * [XIAOMI] §1 and §2 and [NOVITA] (GLM-4.7 FP8); the pages give no bit layout. */
double orc_e4m3_value(uint32_t code) {
  const uint32_t sign = (code >> 7) & 1u, exp = (code >> 3) & 15u, man = code & 7u;
  double mag;
  if (exp == 15 && man == 7) return NAN;
  if (exp == 0)
    mag = ldexp((double)man / 8.0, 1 - 7);
  else
    mag = ldexp(1.0 + (double)man / 8.0, (int)exp - 7);
  return sign ? -mag : mag;
}

/* Round-to-nearest-even onto a format's non-negative grid: among codes 0..max_code (whose
 * values increase with the code) pick the one nearest to t; on an exact tie pick the even
 * code; t beyond the largest value saturates to it. */
static uint32_t rne_on_grid(double t, uint32_t max_code, double (*value)(uint32_t)) {
  if (!(t > 0.0)) return 0;
  if (t >= value(max_code)) return max_code;
  uint32_t lo = 0, hi = max_code; /* invariant: value(lo) <= t < value(hi) */
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (value(mid) <= t) lo = mid; else hi = mid;
  }
  const double dlo = t - value(lo), dhi = value(hi) - t;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

uint32_t orc_e2m1_rne(double t) { return rne_on_grid(fabs(t), 7, orc_e2m1_value); }
uint32_t orc_e4m3_rne(double t) { return rne_on_grid(fabs(t), 0x7E, orc_e4m3_value); }

/* bf16 (8-bit significand, fp32 exponent range), round to nearest even from fp64. */
uint16_t orc_bf16_from_double(double d) {
  if (isnan(d)) return 0x7FC0;
  const uint16_t sign = signbit(d) ? 0x8000 : 0;
  double a = fabs(d);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1): floor(log2 a) = e - 1 */
  int qexp = (e - 1) - 7;     /* spacing of bf16 values at a's binade */
  if (qexp < -133) qexp = -133; /* subnormal spacing 2^-133 */
  const double n = nearbyint(ldexp(a, -qexp)); /* default rounding mode: ties to even */
  const double r = ldexp(n, qexp);
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
  const float f = (float)r;   /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

static double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ---- quantizers ---------------------------------------------------------------------------
 * MXFP4 ([XIAOMI] §2 "QAT를 적용한 MXFP4": 32 values per block under a shared exponent).
 * Blocks run along K (the contiguous axis of each row).  Per the MX specification:
 *   X = floor(log2(amax)) - emax(E2M1), emax = 2, clamped to the E8M0 range [-127, 127];
 *   an all-zero block takes X = -127;  element code = RNE(|v| / 2^X) with saturation at 6,
 *   sign kept (so -0 gives code 8);  scale byte = X + 127.
 * A block holding a non-finite value gets scale 0xFF (NaN) and all-zero codes. */
int64_t orc_quant_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s) {
  int64_t nonfinite = 0;
  const int64_t nblk = cols / 32;
#pragma omp parallel for num_threads(g_threads) reduction(+ : nonfinite) schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nblk; ++b) {
      const float* v = w + r * cols + b * 32;
      uint8_t* qb = q + r * (cols / 2) + b * 16;
      int64_t bad = 0;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        if (!isfinite(v[i])) { ++bad; continue; }
        if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
      }
      if (bad) {
        nonfinite += bad;
        s[r * nblk + b] = 0xFF;
        memset(qb, 0, 16);
        continue;
      }
      int X;
      if (amax == 0.0) {
        X = -127;
      } else {
        int e;
        frexp(amax, &e);
        X = (e - 1) - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
      }
      s[r * nblk + b] = (uint8_t)(X + 127);
      for (int i = 0; i < 32; i += 2) {
        uint32_t c[2];
        for (int j = 0; j < 2; ++j) {
          const double t = ldexp(fabs((double)v[i + j]), -X);
          c[j] = orc_e2m1_rne(t) | (signbit(v[i + j]) ? 8u : 0u);
        }
        qb[i / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  }
  return nonfinite;
}

/* Block-scaled FP8: one fp32 scale per 128x128 block of [rows][K] (the FP8 expert format of
 * the GLM-4.7 deployment, [NOVITA]; the block shape is the workload's).  Reading:
 *   s = fp32(amax / 448)  (1 for an all-zero block);   t = fp32(v / s);
 *   code = sign | RNE_E4M3(|t|), saturating at 448.
 * Both quotients are correctly rounded fp32 divisions; rounding the fp64 quotient of two
 * fp32 numbers to fp32 gives exactly that.  A block holding a non-finite value gets a NaN
 * scale and all-NaN codes (0x7F).
 * Blocks tile the matrix from its first row and column; when a side is not a multiple of 128
 * (one tensor-parallel rank's slice of the GLM intermediate, 1536 / 8 = 192, [NOVITA] §1) the
 * last block along it covers the remaining rows or columns only.  Scales are
 * [ceil(rows/128)][ceil(cols/128)]. */
int64_t orc_quant_fp8_b128(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s) {
  int64_t nonfinite = 0;
  const int64_t brs = (rows + 127) / 128, bcs = (cols + 127) / 128;
#pragma omp parallel for num_threads(g_threads) reduction(+ : nonfinite) schedule(static) collapse(2)
  for (int64_t br = 0; br < brs; ++br) {
    for (int64_t bc = 0; bc < bcs; ++bc) {
      const int64_t r1 = br * 128 + 128 < rows ? br * 128 + 128 : rows;
      const int64_t c1 = bc * 128 + 128 < cols ? bc * 128 + 128 : cols;
      int64_t bad = 0;
      double amax = 0.0;
      for (int64_t r = br * 128; r < r1; ++r)
        for (int64_t c = bc * 128; c < c1; ++c) {
          const float v = w[r * cols + c];
          if (!isfinite(v)) { ++bad; continue; }
          if (fabs((double)v) > amax) amax = fabs((double)v);
        }
      if (bad) {
        nonfinite += bad;
        s[br * bcs + bc] = NAN;
        for (int64_t r = br * 128; r < r1; ++r)
          memset(q + r * cols + bc * 128, 0x7F, (size_t)(c1 - bc * 128));
        continue;
      }
      const float sc = (amax == 0.0) ? 1.0f : (float)(amax / 448.0);
      s[br * bcs + bc] = sc;
      for (int64_t r = br * 128; r < r1; ++r)
        for (int64_t c = bc * 128; c < c1; ++c) {
          const float v = w[r * cols + c];
          const float t = (float)((double)v / (double)sc);
          q[r * cols + c] = (uint8_t)(orc_e4m3_rne((double)t) | (signbit(v) ? 0x80u : 0u));
        }
    }
  }
  return nonfinite;
}

/* Live FP8 activation quantization, the W8A8 variant ([SIONIC], the table under "무엇을
 * 해결하려는가" and idea 1: the activations are quantized to FP8 inside the expert GEMM rather
 * than by a kernel of their own; idea 3: doing so changes the model's outputs, a fidelity cost
 * that must be measured).  The pages fix neither the block nor the scale of the activations;
 * reading: the recipe of the FP8 weights, over 128 consecutive values along K of one token's
 * activation row (the K extent of one weight scale block):
 *   s = fp32(amax / 448)  (1 for an all-zero block);   code = sign | RNE_E4M3(fp32(v / s)),
 * saturating at 448; a block holding a non-finite value gets a NaN scale and codes 0x7F.
 * The input is fp32 (the caller widens bf16 exactly or rounds an fp64 value once). */
int64_t orc_quant_act_fp8(const float* v, int64_t n, uint8_t* q, float* s) {
  int64_t nonfinite = 0;
  for (int64_t b = 0; b < n / 128; ++b) {
    const float* vb = v + b * 128;
    int64_t bad = 0;
    double amax = 0.0;
    for (int64_t i = 0; i < 128; ++i) {
      if (!isfinite(vb[i])) { ++bad; continue; }
      if (fabs((double)vb[i]) > amax) amax = fabs((double)vb[i]);
    }
    if (bad) {
      nonfinite += bad;
      s[b] = NAN;
      memset(q + b * 128, 0x7F, 128);
      continue;
    }
    const float sc = (amax == 0.0) ? 1.0f : (float)(amax / 448.0);
    s[b] = sc;
    for (int64_t i = 0; i < 128; ++i) {
      const float t = (float)((double)vb[i] / (double)sc);
      q[b * 128 + i] = (uint8_t)(orc_e4m3_rne((double)t) | (signbit(vb[i]) ? 0x80u : 0u));
    }
  }
  return nonfinite;
}

/* In place: v[i] <- the value of its W8A8 activation code, code * scale, exact in fp64.  The
 * fp64 inputs are rounded to fp32 first (nearest even), the precision the activation is
 * carried in between the two projections. */
static void act_fake_quant(double* v, int64_t n) {
  float* f = (float*)calloc((size_t)n, sizeof(float));
  uint8_t* q = (uint8_t*)malloc((size_t)n);
  float* s = (float*)malloc(sizeof(float) * (size_t)(n / 128));
  for (int64_t i = 0; i < n; ++i) f[i] = (float)v[i];
  orc_quant_act_fp8(f, n, q, s);
  for (int64_t i = 0; i < n; ++i) v[i] = orc_e4m3_value(q[i]) * (double)s[i / 128];
  free(s);
  free(q);
  free(f);
}

/* Dequantized value of element (r, c) of a packed [rows][K] matrix: code value times the
 * block scale, exact in fp64. */
static double dq_at(int32_t wfmt, const uint8_t* q, const void* s, int64_t K, int64_t r,
                    int64_t c) {
  if (wfmt == ORC_WFMT_MXFP4) {
    const uint8_t byte = q[r * (K / 2) + c / 2];
    const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 15u);
    const uint8_t sb = ((const uint8_t*)s)[r * (K / 32) + c / 32];
    return orc_e2m1_value(code) * orc_e8m0_value(sb);
  }
  const float sc = ((const float*)s)[(r / 128) * ((K + 127) / 128) + c / 128];
  return orc_e4m3_value(q[r * K + c]) * (double)sc;
}

void orc_dequant(int32_t wfmt, const uint8_t* q, const void* s, int64_t rows, int64_t cols,
                 double* out) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = dq_at(wfmt, q, s, cols, r, c);
}

/* ---- router ---------------------------------------------------------------------------------
 * Sparse top-k routing ([XIAOMI] §1, MoE routing; [SIONIC] "무엇을 해결하려는가", top-8
 * experts per token) with the shared expert fused as the last slot ([NOVITA] §1 shared-expert
 * fusion: top-9 of 161, the shared expert always in the ninth position).  Readings where the
 * pages are silent: the logit is x . Wr_e (+ b_e), accumulated in fp64; experts are ranked by
 * (logit descending, index ascending); the k selected get w = sigmoid(l) / sum of the selected
 * sigmoids; the shared expert (stored index E) gets weight 1 exactly. */
typedef struct { double l; int32_t e; } orc_rank;

static int rank_cmp(const void* a, const void* b) {
  const orc_rank* x = (const orc_rank*)a;
  const orc_rank* y = (const orc_rank*)b;
  if (x->l > y->l) return -1;
  if (x->l < y->l) return 1;
  return (x->e < y->e) ? -1 : (x->e > y->e);
}

void orc_route(const uint16_t* x, int32_t M, int32_t H, const float* wr, const float* b,
               int32_t E, int32_t k, int32_t has_shared, int32_t* ids, double* w,
               double* logits, double* gap) {
  const int32_t S = k + (has_shared ? 1 : 0);
  orc_rank* order = (orc_rank*)malloc(sizeof(orc_rank) * (size_t)E);
  for (int32_t t = 0; t < M; ++t) {
    double* lt = logits + (int64_t)t * E;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h)
        acc += bf16_value(x[(int64_t)t * H + h]) * (double)wr[(int64_t)e * H + h];
      if (b) acc += (double)b[e];
      lt[e] = acc;
    }
    for (int32_t e = 0; e < E; ++e) { order[e].l = lt[e]; order[e].e = e; }
    qsort(order, (size_t)E, sizeof(orc_rank), rank_cmp);
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) sum += 1.0 / (1.0 + exp(-order[j].l));
    for (int32_t j = 0; j < k; ++j) {
      ids[t * S + j] = order[j].e;
      w[t * S + j] = (1.0 / (1.0 + exp(-order[j].l))) / sum;
    }
    if (has_shared) {
      ids[t * S + k] = E;
      w[t * S + k] = 1.0;
    }
    gap[t] = (k < E) ? order[k - 1].l - order[k].l : INFINITY;
  }
  free(order);
}

/* ---- expert FFN and combine ---------------------------------------------------------------
 * Each selected expert is a SwiGLU FFN ([XIAOMI] §2, MoE expert FFN layers; the gate form is
 * the workload's): g = Wg x, u = Wu x, a = silu(g) * u with silu(z) = z * sigmoid(z),
 * o = Wd a; the token's output is sum_j w_j * o_j over its slots in slot order, the shared
 * expert's slot included ([NOVITA] §1).  Weights enter dequantized (exact), math in fp64.
 * W8A8 (FP8_B128_A8): x and a enter each projection as the values of their activation codes
 * (orc_quant_act_fp8), everything else unchanged. */
void orc_expert_ffn(const orc_experts* L, const uint16_t* x, int32_t M, const int32_t* ids,
                    const float* w, int32_t S, const uint8_t* token_mask, double* y) {
  const int64_t H = L->hidden, I = L->inter;
  double* xd = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  for (int32_t t = 0; t < M; ++t) {
    double* yt = y + (int64_t)t * H;
    if (token_mask && !token_mask[t]) {
      for (int64_t h = 0; h < H; ++h) yt[h] = NAN;
      continue;
    }
    for (int64_t h = 0; h < H; ++h) { xd[h] = bf16_value(x[(int64_t)t * H + h]); yt[h] = 0.0; }
    if (L->wfmt == ORC_WFMT_FP8_B128_A8) act_fake_quant(xd, H);
    for (int32_t j = 0; j < S; ++j) {
      const int32_t e = ids[t * S + j];
      const double wt = (double)w[t * S + j];
      const uint8_t* q13 = L->w13_q[e];
      const void* s13 = L->w13_s[e];
      const uint8_t* q2 = L->w2_q[e];
      const void* s2 = L->w2_s[e];
#pragma omp parallel for num_threads(g_threads) schedule(static)
      for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) g += dq_at(L->wfmt, q13, s13, H, i, h) * xd[h];
        for (int64_t h = 0; h < H; ++h) u += dq_at(L->wfmt, q13, s13, H, I + i, h) * xd[h];
        const double silu = g / (1.0 + exp(-g));
        a[i] = silu * u;
      }
      if (L->wfmt == ORC_WFMT_FP8_B128_A8) act_fake_quant(a, I);
#pragma omp parallel for num_threads(g_threads) schedule(static)
      for (int64_t h = 0; h < H; ++h) {
        double o = 0.0;
        for (int64_t i = 0; i < I; ++i) o += dq_at(L->wfmt, q2, s2, I, h, i) * a[i];
        yt[h] += wt * o;
      }
    }
  }
  free(a);
  free(xd);
}

/* ---- layer stack pieces -------------------------------------------------------------------
 * RMSNorm between layers ([XIAOMI] §1 names RMSNorm among the per-layer operators whose
 * boundaries cost time; form and epsilon are the workload's): r = 1/sqrt(mean(h^2) + eps),
 * out = bf16((h * r) * gamma).  Residual stream ([XIAOMI] §2 "MoE의 통찰"): h' = bf16(h + y). */
void orc_rmsnorm(const uint16_t* h, int32_t M, int32_t H, const float* gamma, double eps,
                 uint16_t* out) {
  for (int32_t t = 0; t < M; ++t) {
    double ss = 0.0;
    for (int32_t i = 0; i < H; ++i) {
      const double v = bf16_value(h[(int64_t)t * H + i]);
      ss += v * v;
    }
    const double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int32_t i = 0; i < H; ++i)
      out[(int64_t)t * H + i] =
          orc_bf16_from_double((bf16_value(h[(int64_t)t * H + i]) * r) * (double)gamma[i]);
  }
}

void orc_residual(const uint16_t* h, const double* y, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(bf16_value(h[i]) + y[i]);
}

/* ---- verify-acceptance of a speculative block ----------------------------------------------
 * [XIAOMI] §3, the speculative-decoding premise: a draft proposes K tokens, the backbone scores
 * all of them in one forward, and a rejection-sampling step accepts a prefix of them without
 * changing the output distribution (so a forward yields about alpha*K tokens).  [SIONIC] idea 3:
 * the main model confirms at once the leading draft tokens that agree with it (its figures are
 * for greedy decoding).  The pages print no formulas; reading: the standard speculative-sampling
 * rule, written out below.
 * Row i of L (fp32 logits [K+1][V], i = 0..K) scores the token that follows the prefix and the
 * first i draft tokens.  p_i = softmax(L[i]) in fp64: m_i = max, Z_i = sum over x in index
 * order of exp(L[i][x] - m_i).
 * Greedy (Q == NULL): g_i = argmax L[i] (lowest index on ties); d_i is accepted while
 *   d_i == g_i; the token after the accepted prefix is g_n.
 * Sampling: d_i is accepted iff u_i * q_i(d_i) < p_i(d_i) (q_i = Q[i], fp64, u_i in [0,1)).
 *   At the first rejection j the next token is drawn from r(x) = max(0, p_j(x) - q_j(x)), or
 *   from p_j if r sums to 0; when all K are accepted it is drawn from p_K.  A draw from weights
 *   w with total T (index order) takes the smallest x whose inclusive prefix sum exceeds
 *   u_K * T.
 * A draft token outside [0, V) is never accepted.  Logits are finite or -inf, at least one
 * finite per row.
 * out[0..n-1] = the accepted draft tokens, out[n] = the drawn (or argmax) token; returns n + 1.
 * margin (nullable, two values): the smallest relative distance to its threshold of an accept
 * test taken (|u q - p| / max(p, u q)), then of the draw (min(t - C(x-1), C(x) - t) / T); +inf
 * when there is none. */
static void vrow_stats(const float* l, int32_t V, double* m, double* Z, int32_t* am) {
  int32_t a = 0;
  for (int32_t x = 1; x < V; ++x)
    if (l[x] > l[a]) a = x;
  const double mx = (double)l[a];
  double z = 0.0;
  for (int32_t x = 0; x < V; ++x) z += exp((double)l[x] - mx);
  *m = mx;
  *Z = z;
  *am = a;
}

static void note_margin(double* margin, double d) {
  if (margin && d < *margin) *margin = d;
}

/* Smallest x with prefix sum of w (index order) > t; w has total T = that sum over all x. */
static int32_t vdraw(const double* w, int32_t V, double t, double T, double* margin) {
  double c = 0.0;
  for (int32_t x = 0; x < V; ++x) {
    const double prev = c;
    c += w[x];
    if (c > t) {
      note_margin(margin, fmin(t - prev, c - t) / T);
      return x;
    }
  }
  return V - 1; /* not reached: t = u*T < T */
}

int32_t orc_verify(const float* L, const float* Q, const int32_t* d, const float* u, int32_t K,
                   int32_t V, int32_t* out, double* margin) {
  if (margin) margin[0] = margin[1] = INFINITY;
  double* m = (double*)malloc(sizeof(double) * (size_t)(K + 1));
  double* Z = (double*)malloc(sizeof(double) * (size_t)(K + 1));
  int32_t* am = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
  for (int32_t i = 0; i <= K; ++i) vrow_stats(L + (int64_t)i * V, V, &m[i], &Z[i], &am[i]);
  int32_t n = 0;
  if (!Q) {
    while (n < K && d[n] == am[n]) ++n;
    for (int32_t i = 0; i < n; ++i) out[i] = d[i];
    out[n] = am[n];
  } else {
    int32_t j = K;
    for (int32_t i = 0; i < K; ++i) {
      const int32_t t = d[i];
      int accept = 0;
      if (t >= 0 && t < V) {
        const double p = exp((double)L[(int64_t)i * V + t] - m[i]) / Z[i];
        const double uq = (double)u[i] * (double)Q[(int64_t)i * V + t];
        accept = uq < p;
        const double den = fmax(p, uq);
        if (den > 0) note_margin(margin, fabs(p - uq) / den);  /* margin[0] */
      }
      if (!accept) { j = i; break; }
    }
    n = j;
    for (int32_t i = 0; i < n; ++i) out[i] = d[i];
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    const float* lj = L + (int64_t)j * V;
    double T = 0.0;
    if (j < K) {
      const float* qj = Q + (int64_t)j * V;
      for (int32_t x = 0; x < V; ++x) {
        const double r = exp((double)lj[x] - m[j]) / Z[j] - (double)qj[x];
        w[x] = r > 0.0 ? r : 0.0;
        T += w[x];
      }
    }
    if (j == K || T == 0.0) {
      T = 0.0;
      for (int32_t x = 0; x < V; ++x) {
        w[x] = exp((double)lj[x] - m[j]);
        T += w[x];
      }
    }
    out[n] = vdraw(w, V, (double)u[K] * T, T, margin ? margin + 1 : NULL);
    free(w);
  }
  free(am);
  free(Z);
  free(m);
  return n + 1;
}

/* ---- attention-side pre-norms: fused QK-norm + RoPE --------------------------------------
 * [NOVITA] §2 (QKNorm fusion): the head-wise RMSNorm of Q and K and the rotary position
 * embedding run as one kernel; in the GLM4-MoE variant only half of each head's dimensions are
 * rotated.  [XIAOMI] §1 lists RMSNorm and RoPE among the per-layer operators whose boundaries
 * cost time at high token rates.  The pages give no formulas; readings:
 *   per token t and head h (q heads [0, nq) use gamma_q, k heads [nq, nh) gamma_k), x = the
 *   head's hd bf16 values:  r = 1/sqrt(sum(x^2)/hd + eps);  n_k = (x_k * r) * gamma_k;
 *   rotary on the first rot dimensions, pairs (i, i + rot/2) for i < rot/2 (the half-split
 *   pairing): angle = pos_t * theta^(-2i/rot), c = cos(angle), s = sin(angle),
 *   y_i = n_i c - n_{i+rot/2} s,  y_{i+rot/2} = n_{i+rot/2} c + n_i s;  dimensions >= rot keep n.
 * All in fp64; y_f64 (nullable) receives the unrounded values, y_bf16 the values rounded once.
 * Token t's heads start at x + t * stride (elements); head h at offset h * hd. */
void orc_qk_norm_rope(const uint16_t* x, int32_t M, int32_t nq, int32_t nh, int32_t hd,
                      int64_t stride, const int32_t* pos, const float* gq, const float* gk,
                      double eps, double theta, int32_t rot, double* y_f64, uint16_t* y_bf16) {
  double* n = (double*)malloc(sizeof(double) * (size_t)hd);
  for (int32_t t = 0; t < M; ++t) {
    for (int32_t h = 0; h < nh; ++h) {
      const uint16_t* xh = x + (int64_t)t * stride + (int64_t)h * hd;
      const float* g = h < nq ? gq : gk;
      double ss = 0.0;
      for (int32_t k = 0; k < hd; ++k) ss += bf16_value(xh[k]) * bf16_value(xh[k]);
      const double r = 1.0 / sqrt(ss / (double)hd + eps);
      for (int32_t k = 0; k < hd; ++k) n[k] = (bf16_value(xh[k]) * r) * (double)g[k];
      const int64_t o = ((int64_t)t * nh + h) * hd;
      for (int32_t k = 0; k < hd; ++k) {
        double y = n[k];
        if (k < rot) {
          const int32_t half = rot / 2, i = k < half ? k : k - half;
          const double ang = (double)pos[t] * pow(theta, -2.0 * (double)i / (double)rot);
          const double c = cos(ang), sn = sin(ang);
          y = k < half ? n[k] * c - n[k + half] * sn : n[k] * c + n[k - half] * sn;
        }
        if (y_f64) y_f64[o + k] = y;
        y_bf16[o + k] = orc_bf16_from_double(y);
      }
    }
  }
  free(n);
}
