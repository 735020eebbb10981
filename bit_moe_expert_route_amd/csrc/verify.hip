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
// Structure (HBM-bound: the logits are read once, 4 bytes per value and row):
//   stats kernel: one workgroup per 2048-value chunk of every row writes the chunk's max, its
//     lowest argmax and its fp64 sum of exp(l - chunk max).  The last workgroup to finish (a
//     device-scope counter) merges them per row, takes the accept decisions in parallel (one
//     thread per draft position), and either finishes (greedy, or every draft accepted: the
//     bonus token is drawn by a search over the chunk sums, then inside the chosen chunk) or
//     records the rejected position j.
//   residual kernel (sampling only): with a rejection at j, one workgroup per chunk of row j
//     sums max(0, p_j - q_j); the last one draws the token the same way.  Otherwise it returns
//     at once.
// Decisions are taken in fp64 from fp32 logits and draft probabilities.
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

// The last workgroup of a grid to arrive at `counter` returns true (after an acquire fence, so
// every other workgroup's earlier stores are visible to all its threads).  Thread 0 made this
// workgroup's own results visible first.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, uint32_t total, int* si) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    si[2] = atomicAdd(counter, 1u) == total - 1;
  }
  __syncthreads();
  const bool last = si[2] != 0;
  if (last) __threadfence();
  return last;
}

// ---- the weights of a draw ------------------------------------------------------------------

enum WeightKind { kTarget = 0, kResidual = 1 };

// Weight of value x of row `row` (0 beyond V): exp(l - m) (kTarget, unnormalized) or
// max(0, exp(l - m) / Z - q) (kResidual).
__device__ __forceinline__ double draw_weight(const VerifyArgs& a, int row, int x, int kind,
                                              double m, double Z) {
  if (x >= a.V) return 0.0;
  const double e = exp((double)a.L[(int64_t)row * a.V + x] - m);
  if (kind == kTarget) return e;
  const double r = e / Z - (double)a.Q[(int64_t)row * a.V + x];
  return r > 0.0 ? r : 0.0;
}

// Draw from row `row` with a kind of weight whose per-chunk totals are chunk_w(c): the chunk
// search runs over the chunk totals in rounds of kVChunk chunks, then the value search inside
// the chosen chunk.  Rounding can leave the target beyond the last prefix sum; the draw then
// takes the last chunk / value with a positive weight.  Called by one whole workgroup.
template <typename ChunkW>
__device__ int draw_token(const VerifyArgs& a, int row, int kind, double m, double Z,
                          double total, ChunkW chunk_w, double u, double* sd, int* si) {
  const double target = u * total;
  double carry = 0.0;
  int cstar = -1, clast = -1;
  double base = 0.0;
  for (int c0 = 0; c0 < a.nch && cstar < 0; c0 += kVChunk) {
    double w[kVPer];
#pragma unroll
    for (int k = 0; k < kVPer; ++k) {
      const int c = c0 + kVPer * (int)threadIdx.x + k;
      w[k] = c < a.nch ? chunk_w(c) : 0.0;
    }
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
    for (int c = (int)threadIdx.x; c < cstar; c += kVT) t += chunk_w(c);
    base = block_sum(t, sd);
  }
  double w[kVPer];
#pragma unroll
  for (int k = 0; k < kVPer; ++k)
    w[k] = draw_weight(a, row, cstar * kVChunk + kVPer * (int)threadIdx.x + k, kind, m, Z);
  double carry2 = base;
  const int f = block_find(w, carry2, target, sd, si);
  if (f >= 0) return cstar * kVChunk + f;
  const int lp = block_last_positive(w, si);
  return cstar * kVChunk + (lp < 0 ? 0 : lp);
}

// ---- kernels -------------------------------------------------------------------------------

// One workgroup per (row, chunk).  VEC: rows start 16-byte aligned (V % 4 == 0), float4 loads.
template <bool VEC>
__global__ __launch_bounds__(kVT) void verify_stats_kernel(VerifyArgs a) {
  __shared__ float sv[kVT / kWave];
  __shared__ int sx[kVT / kWave];
  __shared__ double sd[kVT / kWave];
  __shared__ int si[4];
  __shared__ double rm[kMaxTokens], rz[kMaxTokens];
  __shared__ int ra[kMaxTokens], acc[kMaxTokens];
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
  if (best != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kVPer; ++k) s += exp((double)v[k] - (double)best);
  }
  s = block_sum(s, sd);
  if (threadIdx.x == 0) {
    const int o = row * a.nch + c;
    a.cm[o] = best;
    a.ca[o] = bx;
    a.cs[o] = s;
  }
  const uint32_t total = (uint32_t)((a.K + 1) * a.nch);
  if (!last_arrival(a.st, total, si)) return;

  // ---- decision (the last workgroup) ----
  for (int i = 0; i <= a.K; ++i) {
    float mv = -INFINITY;
    int mx = 0x7FFFFFFF;
    for (int cc = (int)threadIdx.x; cc < a.nch; cc += kVT) {
      const float cv = a.cm[i * a.nch + cc];
      const int cx = a.ca[i * a.nch + cc];
      if (cv > mv || (cv == mv && cx < mx)) { mv = cv; mx = cx; }
    }
    block_argmax(mv, mx, sv, sx);
    double z = 0.0;
    for (int cc = (int)threadIdx.x; cc < a.nch; cc += kVT) {
      const float cv = a.cm[i * a.nch + cc];
      if (cv != -INFINITY) z += a.cs[i * a.nch + cc] * exp((double)cv - (double)mv);
    }
    z = block_sum(z, sd);
    if (threadIdx.x == 0) {
      rm[i] = (double)mv;
      rz[i] = z;
      ra[i] = mx;
      a.rowmz[2 * i] = (double)mv;
      a.rowmz[2 * i + 1] = z;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < a.K) {
    const int dt = a.d[t];
    int ok = 0;
    if (dt >= 0 && dt < a.V) {
      if (a.Q == nullptr) {
        ok = dt == ra[t];
      } else {
        const double p = exp((double)a.L[(int64_t)t * a.V + dt] - rm[t]) / rz[t];
        ok = (double)a.u[t] * (double)a.Q[(int64_t)t * a.V + dt] < p;
      }
    }
    acc[t] = ok;
  }
  __syncthreads();
  int j = a.K;
  for (int i = 0; i < a.K; ++i)
    if (!acc[i]) { j = i; break; }
  if (t < j) a.out[t] = a.d[t];
  if (a.Q == nullptr) {
    if (t == 0) {
      a.out[j] = ra[j];
      *a.count = j + 1;
      a.st[2] = (uint32_t)a.K;  // nothing left for the residual kernel
      a.st[0] = 0;
    }
    return;
  }
  if (j < a.K) {  // the residual kernel draws the token after the rejection
    if (t == 0) {
      a.st[2] = (uint32_t)j;
      a.st[0] = 0;
    }
    return;
  }
  // every draft accepted: the bonus token from p_K
  const int K = a.K, nch = a.nch;
  const double mK = rm[K], zK = rz[K];
  auto chunk_w = [&](int cc) -> double {
    const float cv = a.cm[K * nch + cc];
    return cv == -INFINITY ? 0.0 : a.cs[K * nch + cc] * exp((double)cv - mK);
  };
  const int tok = draw_token(a, K, kTarget, mK, zK, zK, chunk_w, (double)a.u[K], sd, si);
  if (t == 0) {
    a.out[K] = tok;
    *a.count = K + 1;
    a.st[2] = (uint32_t)K;
    a.st[0] = 0;
  }
}

// One workgroup per chunk of the rejected row j (none with no rejection).
__global__ __launch_bounds__(kVT) void verify_residual_kernel(VerifyArgs a) {
  __shared__ double sd[kVT / kWave];
  __shared__ int si[4];
  const int j = (int)a.st[2];  // written by the stats kernel of this call
  if (j >= a.K) return;
  const double mj = a.rowmz[2 * j], zj = a.rowmz[2 * j + 1];
  const int c = blockIdx.x;
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kVPer; ++k)
    s += draw_weight(a, j, c * kVChunk + kVPer * (int)threadIdx.x + k, kResidual, mj, zj);
  s = block_sum(s, sd);
  if (threadIdx.x == 0) a.rmass[c] = s;
  if (!last_arrival(a.st + 1, (uint32_t)a.nch, si)) return;

  double T = 0.0;
  for (int cc = (int)threadIdx.x; cc < a.nch; cc += kVT) T += a.rmass[cc];
  T = block_sum(T, sd);
  const double u = (double)a.u[a.K];
  int tok;
  if (T > 0.0) {
    auto chunk_w = [&](int cc) -> double { return a.rmass[cc]; };
    tok = draw_token(a, j, kResidual, mj, zj, T, chunk_w, u, sd, si);
  } else {  // the residual is empty: draw from p_j
    const int nch = a.nch;
    auto chunk_w = [&](int cc) -> double {
      const float cv = a.cm[j * nch + cc];
      return cv == -INFINITY ? 0.0 : a.cs[j * nch + cc] * exp((double)cv - mj);
    };
    tok = draw_token(a, j, kTarget, mj, zj, zj, chunk_w, u, sd, si);
  }
  if (threadIdx.x == 0) {
    a.out[j] = tok;
    *a.count = j + 1;
    a.st[1] = 0;
    a.st[2] = (uint32_t)a.K;
  }
}

}  // namespace

int verify_chunks(int V) { return (V + kVChunk - 1) / kVChunk; }

hipError_t launch_verify(const VerifyArgs& a, bool vec, hipStream_t stream) {
  const unsigned grid1 = (unsigned)((a.K + 1) * a.nch);
  if (vec)
    hipLaunchKernelGGL(verify_stats_kernel<true>, dim3(grid1), dim3(kVT), 0, stream, a);
  else
    hipLaunchKernelGGL(verify_stats_kernel<false>, dim3(grid1), dim3(kVT), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.Q == nullptr) return err;
  hipLaunchKernelGGL(verify_residual_kernel, dim3((unsigned)a.nch), dim3(kVT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
