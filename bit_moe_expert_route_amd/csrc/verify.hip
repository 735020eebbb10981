// Verify-acceptance of a speculative block: the step after the backbone's verify forward.
//   molayo1419.me Xiaomi 1T page, section 3 ("the speculative-decoding premise"): a draft
//   proposes K tokens, the backbone scores them in one forward, and rejection sampling accepts
//   a prefix of them without changing the output distribution.
//   d9249.github.io "glm-5-2-b300-kernel-mtp-serving", idea 3: the main model confirms at once
//   the leading draft tokens that agree with it.
// The rule (the standard speculative-sampling rule; the pages print none): row i of the target
// logits L [K+1][V] scores the token after the prefix and the first i draft tokens, with
// p_i = softmax(L[i]).
//   greedy:   draft token d_i is accepted while it equals argmax L[i] (lowest index on ties);
//             the next token is argmax L[n].
//   sampling: d_i is accepted iff u_i * q_i(d_i) < p_i(d_i); at the first rejection j the next
//             token is drawn from max(0, p_j - q_j) (from p_j if that sums to 0), after a full
//             accept from p_K.  A draw takes the smallest index whose prefix sum in index order
//             exceeds u_K times the total.
//
// Structure (HBM-bound: the logits are read once, 4 bytes per value and row), stream-ordered
// launches (a kernel boundary makes one grid's results visible to the next; a last-arriving
// workgroup behind per-workgroup device-scope release fences measured 58 us here against a few
// for the boundaries):
//   stats:  one workgroup per 2048-value chunk of every row writes the chunk's max, its lowest
//           argmax and its fp64 sum of exp(l - chunk max).
//   decide: one workgroup merges them per row, takes the accept decisions in parallel (one
//           thread per draft position) and either finishes (greedy, or every draft accepted: the
//           bonus token is drawn by a search over the chunk sums, then inside the chosen chunk)
//           or records the rejected position j.
//   residual mass, residual draw (sampling only): with a rejection at j, one workgroup per chunk
//           of row j sums max(0, p_j - q_j), then one workgroup draws the token the same way.
//           Without one they return at once.
// Arithmetic: the exponentials of the bulk sums (the normalizer Z_i, the residual masses, the
// draw weights) are fp32 (`__expf` of an fp32 difference, relative error about 1e-7), summed in
// fp64; the accept test evaluates exp of its one logit in fp64.  So a decision can differ from
// an all-fp64 evaluation only when it lies within about 1e-6 of its threshold.
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kVT = 256;              // threads per workgroup
constexpr int kVPer = 8;              // values per thread
constexpr int kVChunk = kVT * kVPer;  // values per chunk

// ---- workgroup helpers (256 threads, 4 waves) ---------------------------------------------

// (max, lowest index) over the workgroup; every thread gets the result.
__device__ __forceinline__ void block_argmax(float& v, int& x, float* sv, int* sx) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int ox = __shfl_xor(x, o, kWave);
    if (ov > v || (ov == v && ox < x)) { v = ov; x = ox; }
  }
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) { sv[w] = v; sx[w] = x; }
  __syncthreads();
  v = sv[0];
  x = sx[0];
#pragma unroll
  for (int i = 1; i < kVT / kWave; ++i)
    if (sv[i] > v || (sv[i] == v && sx[i] < x)) { v = sv[i]; x = sx[i]; }
}

// Sum over the workgroup in a fixed order; every thread gets the result.
__device__ __forceinline__ double block_sum(double v, double* sd) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) sd[w] = v;
  __syncthreads();
  double s = sd[0];
#pragma unroll
  for (int i = 1; i < kVT / kWave; ++i) s += sd[i];
  return s;
}

// Thread t holds the weights of positions kVPer*t + k (k < kVPer) of a range of kVChunk
// positions.  Returns, to every thread, the first position with a positive weight whose prefix
// sum (index order, plus `carry`) exceeds `target`, or -1; `carry` becomes carry + the range's
// total.  (In exact arithmetic the first crossing always has a positive weight; requiring it
// keeps a zero-probability value from being drawn when rounding puts the target below `carry`.)
__device__ __forceinline__ int block_find(const double (&w)[kVPer], double& carry, double target,
                                          double* sd, int* si) {
  double incl[kVPer];
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < kVPer; ++k) { run += w[k]; incl[k] = run; }
  // inclusive scan of the thread totals: within the wave, then across the 4 waves
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  double scan = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double up = __shfl_up(scan, o, kWave);
    if (lane >= o) scan += up;
  }
  __syncthreads();
  if (lane == kWave - 1) sd[wv] = scan;
  if (threadIdx.x == 0) si[0] = 0x7FFFFFFF;
  __syncthreads();
  double before = carry;
  for (int i = 0; i < wv; ++i) before += sd[i];
  before += scan - run;  // exclusive prefix of this thread
  int found = 0x7FFFFFFF;
#pragma unroll
  for (int k = kVPer - 1; k >= 0; --k)
    if (w[k] > 0.0 && before + incl[k] > target) found = kVPer * (int)threadIdx.x + k;
  if (found != 0x7FFFFFFF) atomicMin(&si[0], found);
  double total = 0.0;
#pragma unroll
  for (int i = 0; i < kVT / kWave; ++i) total += sd[i];
  __syncthreads();
  const int r = si[0];
  carry += total;
  return r == 0x7FFFFFFF ? -1 : r;
}

// Last position with a positive weight in the range, or -1 (every thread gets the result).
__device__ __forceinline__ int block_last_positive(const double (&w)[kVPer], int* si) {
  if (threadIdx.x == 0) si[1] = -1;
  __syncthreads();
  int last = -1;
#pragma unroll
  for (int k = 0; k < kVPer; ++k)
    if (w[k] > 0.0) last = kVPer * (int)threadIdx.x + k;
  if (last >= 0) atomicMax(&si[1], last);
  __syncthreads();
  return si[1];
}

// Merge the (max, lowest argmax, sum of exp(l - max)) summary of one set of values into
// another's; -inf maxima are empty sets.  Without SUM only (max, argmax).  The rescaling
// factors are fp32 exponentials like the sums they scale.
template <bool SUM>
__device__ __forceinline__ void merge_stats(float& mv, int& mx, double& z, float mv2, int mx2,
                                            double z2) {
  if (mv2 == -INFINITY) return;
  if (mv == -INFINITY) {
    mv = mv2;
    mx = mx2;
    if constexpr (SUM) z = z2;
  } else if (mv2 > mv) {
    if constexpr (SUM) z = z * (double)__expf(mv - mv2) + z2;
    mv = mv2;
    mx = mx2;
  } else {
    if constexpr (SUM) z += z2 * (double)__expf(mv2 - mv);
    if (mv2 == mv && mx2 < mx) mx = mx2;
  }
}

// ---- the weights of a draw ------------------------------------------------------------------

enum WeightKind { kTarget = 0, kResidual = 1 };

// Weights of the kVPer consecutive values x0 + k of row `row` (0 beyond V): exp(l - m)
// (kTarget, unnormalized) or max(0, exp(l - m) / Z - q) (kResidual).  The loads are
// unconditional, their index clamped into the row, so that all of them are in flight together
// (a load under a branch is waited for inside it).
template <int KIND>
__device__ __forceinline__ void draw_weights(const VerifyArgs& a, int row, int x0, double m,
                                             double Z, double (&w)[kVPer]) {
  const int64_t rb = (int64_t)row * a.V;
  float l[kVPer], q[kVPer];
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    const int x = x0 + k < a.V ? x0 + k : a.V - 1;
    l[k] = a.L[rb + x];
    if constexpr (KIND == kResidual) q[k] = a.Q[rb + x];
  }
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    double r = (double)__expf(l[k] - (float)m);
    if constexpr (KIND == kResidual) {
      r = r / Z - (double)q[k];
      r = r > 0.0 ? r : 0.0;
    }
    w[k] = x0 + k < a.V ? r : 0.0;
  }
}

// Per-chunk totals of the same weights: the residual masses (kResidual), or the chunk's
// exp-sum rescaled to the row maximum m (kTarget; 0 for an all -inf chunk).
template <int KIND>
__device__ __forceinline__ double chunk_weight(const VerifyArgs& a, int row, int c, double m) {
  if constexpr (KIND == kResidual) {
    return a.rmass[c];
  } else {
    const float cm = a.cm[row * a.nch + c];
    const double cz = a.cs[row * a.nch + c];
    return cm == -INFINITY ? 0.0 : cz * exp((double)cm - m);
  }
}

// The totals of chunks c0 + k (0 beyond nch); every load is issued before any is used.
template <int KIND>
__device__ __forceinline__ void chunk_weights(const VerifyArgs& a, int row, int c0, double m,
                                              double (&w)[kVPer]) {
  float cm[kVPer];
  double cz[kVPer];
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    const int c = c0 + k < a.nch ? c0 + k : a.nch - 1;
    if constexpr (KIND == kResidual) {
      cz[k] = a.rmass[c];
    } else {
      cm[k] = a.cm[row * a.nch + c];
      cz[k] = a.cs[row * a.nch + c];
    }
  }
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    opaque(cz[k]);
    if constexpr (KIND == kTarget) asm volatile("" : "+v"(cm[k]));
  }
#pragma unroll
  for (int k = 0; k < kVPer; ++k) {
    double v = cz[k];
    if constexpr (KIND == kTarget) v = cm[k] == -INFINITY ? 0.0 : v * exp((double)cm[k] - m);
    w[k] = c0 + k < a.nch ? v : 0.0;
  }
}

// Draw from row `row` by the weights of KIND, whose per-chunk totals chunk_weights gives: the
// chunk search runs over the chunk totals in rounds of kVChunk chunks, then the value search
// inside the chosen chunk.  Rounding can leave the target beyond the last prefix sum; the draw
// then takes the last chunk / value with a positive weight.  Called by one whole workgroup.
template <int KIND>
__device__ int draw_token(const VerifyArgs& a, int row, double m, double Z, double total,
                          double u, double* sd, int* si) {
  const double target = u * total;
  double carry = 0.0;
  int cstar = -1, clast = -1;
  double base = 0.0;
  for (int c0 = 0; c0 < a.nch && cstar < 0; c0 += kVChunk) {
    double w[kVPer];
    chunk_weights<KIND>(a, row, c0 + kVPer * (int)threadIdx.x, m, w);
    const double before = carry;
    const int f = block_find(w, carry, target, sd, si);
    const int lp = block_last_positive(w, si);
    if (lp >= 0) clast = c0 + lp;
    if (f >= 0) {
      cstar = c0 + f;
      // prefix before the chosen chunk, in the same order as the search
      double wb[kVPer];
#pragma unroll
      for (int k = 0; k < kVPer; ++k) {
        const int c = c0 + kVPer * (int)threadIdx.x + k;
        wb[k] = c < cstar ? w[k] : 0.0;
      }
      double t = 0.0;
#pragma unroll
      for (int k = 0; k < kVPer; ++k) t += wb[k];
      base = before + block_sum(t, sd);
    }
  }
  if (cstar < 0) {  // target at or beyond the searched total
    cstar = clast < 0 ? 0 : clast;
    double t = 0.0;
    for (int c = (int)threadIdx.x; c < cstar; c += kVT) t += chunk_weight<KIND>(a, row, c, m);
    base = block_sum(t, sd);
  }
  double w[kVPer];
  draw_weights<KIND>(a, row, cstar * kVChunk + kVPer * (int)threadIdx.x, m, Z, w);
  double carry2 = base;
  const int f = block_find(w, carry2, target, sd, si);
  if (f >= 0) return cstar * kVChunk + f;
  const int lp = block_last_positive(w, si);
  return cstar * kVChunk + (lp < 0 ? 0 : lp);
}

// ---- kernels -------------------------------------------------------------------------------

// One workgroup per (row, chunk).  VEC: rows start 16-byte aligned (V % 4 == 0), float4 loads.
// SAMPLE: also the exp-sums (greedy needs only the argmax).
template <bool VEC, bool SAMPLE>
__global__ __launch_bounds__(kVT) void verify_stats_kernel(VerifyArgs a) {
  __shared__ float sv[kVT / kWave];
  __shared__ int sx[kVT / kWave];
  __shared__ double sd[kVT / kWave];
  const int row = blockIdx.x / a.nch, c = blockIdx.x % a.nch;
  const float* lrow = a.L + (int64_t)row * a.V;
  const int x0 = c * kVChunk;
  float v[kVPer];
  int xi[kVPer];
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < kVPer / 4; ++k) {
      const int x = x0 + 4 * (int)threadIdx.x + 4 * kVT * k;
      float4 f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (x < a.V) f = *reinterpret_cast<const float4*>(lrow + x);  // V % 4 == 0: whole float4
      v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
#pragma unroll
      for (int e = 0; e < 4; ++e) xi[4 * k + e] = x + e;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kVPer; ++k) {
      const int x = x0 + (int)threadIdx.x + kVT * k;
      v[k] = x < a.V ? lrow[x] : -INFINITY;
      xi[k] = x;
    }
  }
  // chunk max and its lowest index (values beyond V are -inf and never win)
  float best = -INFINITY;
  int bx = 0x7FFFFFFF;
#pragma unroll
  for (int k = 0; k < kVPer; ++k)
    if (xi[k] < a.V && (v[k] > best || (v[k] == best && xi[k] < bx))) { best = v[k]; bx = xi[k]; }
  block_argmax(best, bx, sv, sx);
  double s = 0.0;
  if constexpr (SAMPLE) {
    if (best != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kVPer; ++k) s += (double)__expf(v[k] - best);
    }
    s = block_sum(s, sd);
  }
  if (threadIdx.x == 0) {
    const int o = row * a.nch + c;
    a.cm[o] = best;
    a.ca[o] = bx;
    a.cs[o] = s;
  }
}

// One workgroup: per-row merge, accept decisions, and the bonus draw after a full accept.
// SAMPLE: sampling (greedy merges the argmax only).
template <bool SAMPLE>
__global__ __launch_bounds__(kVT) void verify_decide_kernel(VerifyArgs a) {
  __shared__ double sd[kVT / kWave];
  __shared__ int si[4];
  __shared__ double rm[kMaxTokens], rz[kMaxTokens];
  __shared__ int ra[kMaxTokens], acc[kMaxTokens];
  // per-row merge: wave w takes rows w, w + 4, ... and its lanes the chunks; every lane's loads
  // of all its rows are issued together (one memory latency per 64 chunks)
  constexpr int kWaves = kVT / kWave, kRowsPerWave = kMaxTokens / kWaves;
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  const int t = threadIdx.x;
  // the accept inputs of position t go out first: its draft token, then (once that arrives,
  // while the merge's loads are in flight) the target logit and draft probability it names
  int dt = -1;
  if (t < a.K) dt = a.d[t];
  float lt = 0.0f, qt = 0.0f, ut = 0.0f;
  float mv[kRowsPerWave];
  int mx[kRowsPerWave];
  double z[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) { mv[k] = -INFINITY; mx[k] = 0x7FFFFFFF; z[k] = 0.0; }
  float cv[kRowsPerWave];
  int cx[kRowsPerWave];
  double cz[kRowsPerWave];
  auto load_chunk = [&](int cc) {
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int i = wv + kWaves * k;
      const int o = (i <= a.K ? i : 0) * a.nch + cc;
      cv[k] = i <= a.K ? a.cm[o] : -INFINITY;
      cx[k] = a.ca[o];
      if constexpr (SAMPLE) cz[k] = a.cs[o];
      else cz[k] = 0.0;
    }
  };
  auto merge_chunk = [&]() {
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k)
      merge_stats<SAMPLE>(mv[k], mx[k], z[k], cv[k], cx[k], cz[k]);
  };
  if (lane < a.nch) load_chunk(lane);
  // loads complete in issue order: waiting for d[t] does not wait for the chunk loads
  if (t < a.K && dt >= 0 && dt < a.V && a.Q != nullptr) {
    lt = a.L[(int64_t)t * a.V + dt];
    qt = a.Q[(int64_t)t * a.V + dt];
    ut = a.u[t];
  }
  if (lane < a.nch) merge_chunk();
  for (int cc = lane + kWave; cc < a.nch; cc += kWave) {
    load_chunk(cc);
    merge_chunk();
  }
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float mv2 = __shfl_xor(mv[k], o, kWave);
      const int mx2 = __shfl_xor(mx[k], o, kWave);
      const double z2 = __shfl_xor(z[k], o, kWave);
      merge_stats<SAMPLE>(mv[k], mx[k], z[k], mv2, mx2, z2);
    }
    const int i = wv + kWaves * k;
    if (lane == 0 && i <= a.K) {
      rm[i] = (double)mv[k];
      rz[i] = z[k];
      ra[i] = mx[k];
      a.rowmz[2 * i] = (double)mv[k];
      a.rowmz[2 * i + 1] = z[k];
    }
  }
  __syncthreads();
  if (t < a.K) {
    int ok = 0;
    if (dt >= 0 && dt < a.V) {
      if constexpr (!SAMPLE) {
        ok = dt == ra[t];
      } else {
        const double p = exp((double)lt - rm[t]) / rz[t];
        ok = (double)ut * (double)qt < p;
      }
    }
    acc[t] = ok;
  }
  __syncthreads();
  int j = a.K;
  for (int i = 0; i < a.K; ++i)
    if (!acc[i]) { j = i; break; }
  if (t < j) a.out[t] = a.d[t];
  if constexpr (!SAMPLE) {
    if (t == 0) {
      a.out[j] = ra[j];
      *a.count = j + 1;
    }
    return;
  }
  if (j < a.K) {  // the residual kernels draw the token after the rejection
    if (t == 0) a.st[0] = (uint32_t)j;
    return;
  }
  // every draft accepted: the bonus token from p_K
  const int K = a.K;
  const double mK = rm[K], zK = rz[K];
  const int tok = draw_token<kTarget>(a, K, mK, zK, zK, (double)a.u[K], sd, si);
  if (t == 0) {
    a.out[K] = tok;
    *a.count = K + 1;
    a.st[0] = (uint32_t)K;  // nothing left for the residual kernels
  }
}

// One workgroup per chunk of the rejected row j: its residual mass (nothing without a rejection).
__global__ __launch_bounds__(kVT) void verify_residual_mass_kernel(VerifyArgs a) {
  __shared__ double sd[kVT / kWave];
  const int j = (int)a.st[0];  // written by this call's decide kernel
  if (j >= a.K) return;
  const double mj = a.rowmz[2 * j], zj = a.rowmz[2 * j + 1];
  const int c = blockIdx.x;
  double w[kVPer];
  draw_weights<kResidual>(a, j, c * kVChunk + kVPer * (int)threadIdx.x, mj, zj, w);
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kVPer; ++k) s += w[k];
  s = block_sum(s, sd);
  if (threadIdx.x == 0) a.rmass[c] = s;
}

// One workgroup: the draw after the rejection at j (nothing without one).
__global__ __launch_bounds__(kVT) void verify_residual_draw_kernel(VerifyArgs a) {
  __shared__ double sd[kVT / kWave];
  __shared__ int si[4];
  const int j = (int)a.st[0];
  if (j >= a.K) return;
  const double mj = a.rowmz[2 * j], zj = a.rowmz[2 * j + 1];
  double T = 0.0;
  for (int cc = (int)threadIdx.x; cc < a.nch; cc += kVT) T += a.rmass[cc];
  T = block_sum(T, sd);
  const double u = (double)a.u[a.K];
  int tok;
  if (T > 0.0) {
    tok = draw_token<kResidual>(a, j, mj, zj, T, u, sd, si);
  } else {  // the residual is empty: draw from p_j
    tok = draw_token<kTarget>(a, j, mj, zj, zj, u, sd, si);
  }
  if (threadIdx.x == 0) {
    a.out[j] = tok;
    *a.count = j + 1;
  }
}

}  // namespace

int verify_chunks(int V) { return (V + kVChunk - 1) / kVChunk; }

hipError_t launch_verify(const VerifyArgs& a, bool vec, hipStream_t stream) {
  const unsigned grid1 = (unsigned)((a.K + 1) * a.nch);
  const bool sample = a.Q != nullptr;
  auto stats = vec ? (sample ? verify_stats_kernel<true, true> : verify_stats_kernel<true, false>)
                   : (sample ? verify_stats_kernel<false, true> : verify_stats_kernel<false, false>);
  hipLaunchKernelGGL(stats, dim3(grid1), dim3(kVT), 0, stream, a);
  if (sample)
    hipLaunchKernelGGL(verify_decide_kernel<true>, dim3(1), dim3(kVT), 0, stream, a);
  else
    hipLaunchKernelGGL(verify_decide_kernel<false>, dim3(1), dim3(kVT), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !sample) return err;
  hipLaunchKernelGGL(verify_residual_mass_kernel, dim3((unsigned)a.nch), dim3(kVT), 0, stream,
                     a);
  hipLaunchKernelGGL(verify_residual_draw_kernel, dim3(1), dim3(kVT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
