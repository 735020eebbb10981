// Expert gate/up + SwiGLU with several tokens, on the matrix cores for the experts that several
// (token, slot) pairs selected.
//   d9249.github.io "glm-5-2-b300-kernel-mtp-serving", idea 3: the M tokens of a verify block
//   share one weight stream, so an expert that several of them selected is a small matrix
//   product (rows of the expert times the tokens that chose it), not a set of independent
//   matrix-vector products.
//   molayo1419.me Xiaomi 1T page, section 2: expert FFN weights in MXFP4 (E2M1 values with one
//   E8M0 scale per 32 along the reduction axis).
//   blogs.novita.ai "Optimizing GLM4-MoE for production", section 1: the shared expert is one
//   more slot of the fused MoE; every token selects it.
//
// Why: on the vector path an expert with m pairs costs m passes over its weights, each pass
// reloading another token's activations from L2 (measured on the 1T layer with 16 tokens: 144
// pairs took 266 us of gate/up even when they fell on only 17 experts).  A 16x16x32 bf16 MFMA
// takes 16 weight rows and up to 16 tokens at once, so such an expert costs one pass.
//
// One launch per stage, one workgroup of 8 waves per CU; workgroups [0, Gm) take the
// matrix-core tiles of the experts with 2..16 pairs, the others the vector units of the rest,
// with Gm set by the two parts' costs, so both parts stream at once and share one ramp and
// tail (as two launches the tiles' own ramp and tail cost more than the tiles saved).
//   gate/up (gateup_mix_kernel): a tile is 16 consecutive intermediate indices i0..i0+15 of
//     one expert: its 16 gate and 16 up rows over the whole reduction axis H.  The workgroup's
//     waves split H (wave w takes windows [NWIN*w/8, NWIN*(w+1)/8) of 128 values, with its
//     column's activations of those windows in registers for all tiles of an expert),
//     accumulate 16x16 partial products of gate and up, and leave them in an LDS slot; the wave
//     that arrives last at a tile sums the 8 partials in wave order (so the result does not
//     depend on arrival order), applies SwiGLU and stores a.  Waves do not wait for each other
//     between tiles; a ring of kSlots slots lets them run up to kSlots tiles apart.  The vector
//     part is the workgroup-per-CU gate/up body (gateup_range).
//   down (down_mix_kernel): a tile is 16 rows of W2 over the whole intermediate axis, taken
//     whole by one wave against the expert's a held in LDS; the vector part is the
//     workgroup-per-CU down body.
// MFMA operands (v_mfma_f32_16x16x32_bf16; lane l = 16*g + c, g = l / 16, c = l % 16):
//   A (weights): row c of the tile, the 8 values of reduction positions 8g..8g+7 of the MFMA;
//   B (tokens):  column c = the expert's c-th pair, the same 8 positions;
//   D:           rows 4g..4g+3 of column c, in fp32.
// The reduction axis is permuted so that every lane loads whole 16-byte pieces: in window win
// (positions 128*win .. 128*win+127), lane group g takes the 32 positions 128*win + 32*g ..
// +31, and MFMA j (j = 0..3) the 8 of them at 8*j.  A and B use the same permutation, and a
// dot product does not depend on the order of its terms beyond rounding.
//   MXFP4: the 32 positions of a lane are one scale block; each 8 E2M1 values are decoded with
//          the block's E8M0 scale folded in by v_cvt_scalef32_pk_bf16_fp4, which is exact in
//          bf16 for every scale up to 2^125 (an in-bounds check of all 255 scales and 256 code
//          pairs against the exact products) and 2^125 is the largest the quantizer emits.
//   FP8:   E4M3 decodes exactly to bf16; a window is one 128x128 scale block of the gate rows
//          and one of the up rows (16 rows never straddle a block edge), so each window's
//          product is scaled once in fp32.
#include "ffn_body.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;     // intermediate indices per tile
constexpr int kWinVals = 128;     // reduction values per window (four MFMAs)
constexpr int kMfmaMinPairs = 2;  // experts with 2..16 pairs take the matrix cores
constexpr int kMfmaMaxPairs = 16;
constexpr int kSlots = 3;         // partial-sum slots per workgroup
constexpr int kMfmaThreads = 512;  // 8 waves, two per SIMD (256 registers each)
// The matrix-core kernel runs before the vector one from this many tokens on (with fewer, its
// few tiles cost a launch and save less).
constexpr int kMfmaMinTokens = 8;
// Cost of one tile in the cost-weighted split: gate/up in vector passes over one unit (a tile
// holds 16 units' bytes and streams more slowly), down in quarters of a pass over an 8-row unit
// (a tile holds two units' bytes).
constexpr int kTileCost = 23;
constexpr int kDownTileCost = 11;

template <int NWV>
struct MfmaLds {
  QueueLdsT<NWV> q;
  uint32_t bits_m[NWV][kBitmapWords];
  int base_m[NWV][kBitmapWords];
  f32x4 part[kSlots][NWV][2][kWave];  // [slot][wave][gate, up][lane]
  int arrive[kSlots];
  int slot_tile[kSlots];  // the local tile index the slot takes next
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint32_t bits_of(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Eight E2M1 values (one dword) times the scale sc, as eight bf16 (exact, see above).
__device__ __forceinline__ bf16x8 fp4x8_scaled(uint32_t w, float sc) {
  return as_bf16x8(bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                   bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                   bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                   bits_of(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)));
}

// Eight E4M3 values (two dwords) as eight bf16 (exact).
__device__ __forceinline__ bf16x8 fp8x8_bf16(uint32_t w0, uint32_t w1) {
  bf16x2 a, b, c, d;
  fp8x4_to_bf16(w0, a, b);
  fp8x4_to_bf16(w1, c, d);
  return as_bf16x8(bits_of(a), bits_of(b), bits_of(c), bits_of(d));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Pair index of the n-th set bit of the masks (n < total count).
__device__ __forceinline__ int nth_pair(const uint64_t (&mask)[kPairRegs], int n) {
  int p = 0;
  bool found = false;
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k) {
    const int c = __popcll(mask[k]);
    if (!found && n < c) {
      uint64_t m = mask[k];
      for (int j = 0; j < n; ++j) m &= m - 1;
      p = kWave * k + __builtin_ctzll(m);
      found = true;
    }
    n -= found ? 0 : c;
  }
  return p;
}

// One wave's activations for every tile of one expert: the WMAX windows from w0 of its
// column's token (lane group g: the 32 values at 32*g of each window; windows past the wave's n
// repeat its last one, or w0 when it has none, which is always inside the row).
template <int WMAX>
struct TileX {
  uint4 v[WMAX][4];
};

template <int WMAX>
__device__ __forceinline__ void tile_x_load(const FfnArgs& a, int tok, int w0, int n,
                                            TileX<WMAX>& X) {
  const int g = (threadIdx.x % kWave) >> 4;
  const uint16_t* xr = a.x + (int64_t)tok * a.H + 32 * g;
#pragma unroll
  for (int d = 0; d < WMAX; ++d) {
    const int win = w0 + (d < n ? d : (n > 0 ? n - 1 : 0));
    const uint4* xp = reinterpret_cast<const uint4*>(xr + (int64_t)win * kWinVals);
#pragma unroll
    for (int j = 0; j < 4; ++j) X.v[d][j] = xp[j];
  }
}

// One wave's weights of one tile for HB of its windows, from its window d0: 16 gate and 16 up
// rows from intermediate index i0 of expert e (lane row c).
template <int FMT, int HB>
struct TileW {
  static constexpr int kPiece = FMT == WFMT_MXFP4 ? 1 : 2;  // 16-byte pieces per window
  uint4 g[HB][kPiece], u[HB][kPiece];
  uint32_t sg[HB], su[HB];
};

// Raw buffer loads: one lane offset in a register and the window's offset in a scalar, so a tile
// needs no per-window address registers; the descriptor's byte count bounds every load (a
// load past it returns zero), so the windows past the wave's n (whose products are zeroed) need
// no clamping.  The weights are loaded with the default cache policy: a window reads half of a
// 128-byte line of each of its rows and the next window the other half, which a non-temporal
// load let the cache drop in between (measured slower).
constexpr int kCachePolicy = 0;

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicy);
}

template <int FMT, int HB>
__device__ __forceinline__ void tile_w_load(const FfnArgs& a, int e, int i0, int w0, int n,
                                            int d0, TileW<FMT, HB>& T) {
  constexpr int kPiece = TileW<FMT, HB>::kPiece;
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I;
  const int rb = (int)Fmt<FMT>::row_bytes(H);
  const int ebytes = 2 * I * rb;  // W13 bytes of one expert
  const int ws = w0 + d0;         // first window of this load
  if constexpr (FMT == WFMT_MXFP4) {
    // The E8M0 bytes of windows ws.. of the lane's gate and up rows: the aligned 16-byte blocks
    // that hold them (lane group g takes byte g of each window's word), issued before the
    // weights so that their wait does not wait for the weights.
    constexpr int NB = (4 * HB + 12 + 15) / 16;
    const int sbytes = 2 * I * (H >> 5);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.w13s)) + (int64_t)e * sbytes,
        (short)0, sbytes, kRsrcWord3);
    const int b0 = (4 * ws) & ~15, sh = ws & 3;  // sh: the first window's word in block 0
    u32x4 bg[NB], bu[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      bg[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (i0 + c) * (H >> 5), b0 + 16 * k, 0);
      bu[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (I + i0 + c) * (H >> 5), b0 + 16 * k, 0);
    }
#pragma unroll
    for (int d = 0; d < HB; ++d) {
      // word sh + d of the blocks, sh wave-uniform in 0..3
      uint32_t vg = 0, vu = 0;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int wi = s4 + d;
        if (wi < 4 * NB) {
          vg = sh == s4 ? bg[wi >> 2][wi & 3] : vg;
          vu = sh == s4 ? bu[wi >> 2][wi & 3] : vu;
        }
      }
      T.sg[d] = vg;
      T.su[d] = vu;
    }
  }
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w13) + (int64_t)e * ebytes, (short)0, ebytes, kRsrcWord3);
  const int vg = (i0 + c) * rb + g * 16 * kPiece;  // this lane's piece of its gate row
  const int vu = vg + I * rb;
  (void)n;
#pragma unroll
  for (int d = 0; d < HB; ++d) {
    const int win = ws + d;
#pragma unroll
    for (int p = 0; p < kPiece; ++p) {
      const u32x4 wg = buf_load16(rw, vg + 16 * p, win * 64 * kPiece);
      const u32x4 wu = buf_load16(rw, vu + 16 * p, win * 64 * kPiece);
      T.g[d][p] = make_uint4(wg.x, wg.y, wg.z, wg.w);
      T.u[d][p] = make_uint4(wu.x, wu.y, wu.z, wu.w);
    }
    if constexpr (FMT != WFMT_MXFP4) {
      const float* S = reinterpret_cast<const float*>(a.w13s) +
                       (int64_t)e * scale_elems<FMT>(2 * I, H);
      const int nb = fp8_blocks(H);
      const int wc = win < nb ? win : nb - 1;  // in the scale row (a window past n is zeroed)
      T.sg[d] = __float_as_uint(S[(i0 >> 7) * nb + wc]);
      T.su[d] = __float_as_uint(S[((I + i0) >> 7) * nb + wc]);
    }
  }
}

// The wave's partial products over the HB windows from D0 of its n (into dg, du), in fp32.
// Every window's products are computed, those of a repeated window with a zero scale: a product
// under a branch would pull its loads into the branch and wait for them there.
template <int FMT, int HB, int D0, int WMAX>
__device__ __forceinline__ void tile_mma(const TileW<FMT, HB>& T, const TileX<WMAX>& X, int n,
                                         f32x4& dg, f32x4& du) {
  const int g = (threadIdx.x % kWave) >> 4;
#pragma unroll
  for (int d = 0; d < HB; ++d) {
    constexpr int kLast = WMAX - 1;
    const int dd = D0 + d;
    const bool valid = dd < n;
    const uint4* xw = X.v[dd < kLast ? dd : kLast];
    if constexpr (FMT == WFMT_MXFP4) {
      const float scg = valid ? e8m0_to_f32((T.sg[d] >> (8 * g)) & 0xFFu) : 0.0f;
      const float scu = valid ? e8m0_to_f32((T.su[d] >> (8 * g)) & 0xFFu) : 0.0f;
      const uint32_t wg4[4] = {T.g[d][0].x, T.g[d][0].y, T.g[d][0].z, T.g[d][0].w};
      const uint32_t wu4[4] = {T.u[d][0].x, T.u[d][0].y, T.u[d][0].z, T.u[d][0].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b = as_bf16x8(xw[j].x, xw[j].y, xw[j].z, xw[j].w);
        dg = mfma(fp4x8_scaled(wg4[j], scg), b, dg);
        du = mfma(fp4x8_scaled(wu4[j], scu), b, du);
      }
    } else {
      const uint32_t wg8[8] = {T.g[d][0].x, T.g[d][0].y, T.g[d][0].z, T.g[d][0].w,
                               T.g[d][1].x, T.g[d][1].y, T.g[d][1].z, T.g[d][1].w};
      const uint32_t wu8[8] = {T.u[d][0].x, T.u[d][0].y, T.u[d][0].z, T.u[d][0].w,
                               T.u[d][1].x, T.u[d][1].y, T.u[d][1].z, T.u[d][1].w};
      f32x4 pg = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b = as_bf16x8(xw[j].x, xw[j].y, xw[j].z, xw[j].w);
        pg = mfma(fp8x8_bf16(wg8[2 * j], wg8[2 * j + 1]), b, pg);
        pu = mfma(fp8x8_bf16(wu8[2 * j], wu8[2 * j + 1]), b, pu);
      }
      const float s_g = valid ? __uint_as_float(T.sg[d]) : 0.0f;
      const float s_u = valid ? __uint_as_float(T.su[d]) : 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        dg[v] = __builtin_fmaf(pg[v], s_g, dg[v]);
        du[v] = __builtin_fmaf(pu[v], s_u, du[v]);
      }
    }
  }
}

// The queue of one class of the routed experts: MX = true keeps the experts with
// kMfmaMinPairs..kMfmaMaxPairs pairs, false the others.  cnt: the wave's LDS scratch of
// kMaxPairs words; bits, base: the class queue's own LDS bitmap.
template <bool MX>
__device__ __forceinline__ void class_queue(const WaveQueue& Q, int* cnt, uint32_t* bits,
                                            int* base, int n_pairs, int n_experts,
                                            WaveQueue& C) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < 4; ++j) cnt[4 * lane + j] = 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k)
    if (Q.rank[k] >= 0) atomicAdd(&cnt[Q.rank[k]], 1);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  int v[kPairRegs];
#pragma unroll
  for (int k = 0; k < kPairRegs; ++k) {
    const int m = Q.rank[k] >= 0 ? cnt[Q.rank[k]] : 0;
    const bool mx = m >= kMfmaMinPairs && m <= kMfmaMaxPairs;
    v[k] = mx == MX ? Q.e[k] : -1;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  wave_queue_from(C, bits, base, v, n_pairs, n_experts);
}

// Workgroups of the matrix-core part: the share of the grid that its cost cm takes of cm + cv
// (at least one when there are tiles, and one left for the vector part when it has work).
__device__ __forceinline__ int role_split(int64_t cm, int64_t cv, int G) {
  if (cm <= 0) return 0;
  if (cv <= 0) return G;
  int gm = (int)((cm * G + (cm + cv) / 2) / (cm + cv));
  return gm < 1 ? 1 : (gm > G - 1 ? G - 1 : gm);
}

// The matrix-core tiles [t0, t1) of the experts with 2..16 pairs (queue Qm), by the whole
// workgroup.
template <int FMT, int WMAX>
__device__ __forceinline__ void gateup_tiles(const FfnArgs& a, MfmaLds<kMfmaThreads / kWave>& L,
                                             const WaveQueue& Qm, int t0, int t1) {
  constexpr int NWV = kMfmaThreads / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int I = a.I, S = a.S;
  const int tpe = I / kTileRows;
  if (threadIdx.x < kSlots) {
    L.arrive[threadIdx.x] = 0;
    L.slot_tile[threadIdx.x] = threadIdx.x;
  }
  __syncthreads();
  // ---- matrix-core tiles
  const int nwin = a.H / kWinVals;
  const int w0 = nwin * wave / NWV, n = nwin * (wave + 1) / NWV - w0;
  const int c = lane & 15, g = lane >> 4;
  int cur_q = -1, e = 0, m = 0, pair = 0;
  // kPipe: the wave's windows in two halves of HB; the second half's loads are in flight while
  // the first half's products run, and the next tile's first half while the second half's run.
  // Otherwise (more windows than the registers hold twice) all windows are loaded at the start
  // of each tile.  The activations stay in registers for all tiles of an expert.
  constexpr bool kPipe = WMAX >= 2 && WMAX <= (FMT == WFMT_MXFP4 ? 6 : 4);
  constexpr int HB = kPipe ? (WMAX + 1) / 2 : WMAX;  // first half
  constexpr int HB2 = kPipe ? WMAX - HB : 1;          // second half
  TileX<WMAX> X;
  TileW<FMT, HB> A;
  TileW<FMT, HB2> B;
  auto switch_expert = [&](int q) {
    cur_q = q;
    e = wave_queue_expert(Qm, q);
    uint64_t pm[kPairRegs];
    wave_queue_pairs(Qm, q, pm);
    m = 0;
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) m += __popcll(pm[k]);
    // column c: the expert's c-th pair (columns past m repeat the last and are not stored)
    pair = nth_pair(pm, c < m ? c : m - 1);
    tile_x_load(a, pair / S, w0, n, X);
  };
  if (t0 < t1) {
    switch_expert(t0 / tpe);
    if constexpr (kPipe) tile_w_load(a, e, (t0 % tpe) * kTileRows, w0, n, 0, A);
  }
  for (int t = t0; t < t1; ++t) {
    const int i0 = (t % tpe) * kTileRows;
    const bool more = t + 1 < t1;
    const bool same = more && (t + 1) / tpe == cur_q;
    f32x4 dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kPipe) {
      tile_w_load(a, e, i0, w0, n, HB, B);
      tile_mma<FMT, HB, 0>(A, X, n, dg, du);
      if (same) tile_w_load(a, e, ((t + 1) % tpe) * kTileRows, w0, n, 0, A);
      tile_mma<FMT, HB2, HB>(B, X, n, dg, du);
    } else {
      tile_w_load(a, e, i0, w0, n, 0, A);
      tile_mma<FMT, HB, 0>(A, X, n, dg, du);
    }
    const int lt = t - t0, slot = lt % kSlots;
    if (lane == 0) {
      while (__hip_atomic_load(&L.slot_tile[slot], __ATOMIC_ACQUIRE,
                               __HIP_MEMORY_SCOPE_WORKGROUP) != lt)
        __builtin_amdgcn_s_sleep(1);
    }
    L.part[slot][wave][0][lane] = dg;
    L.part[slot][wave][1][lane] = du;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    int old = 0;
    if (lane == 0) old = atomicAdd(&L.arrive[slot], 1);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == NWV - 1) {  // last to arrive: sum the partials in wave order, SwiGLU, store
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      f32x4 sgt = L.part[slot][0][0][lane], sut = L.part[slot][0][1][lane];
#pragma unroll
      for (int w = 1; w < NWV; ++w) {
        sgt += L.part[slot][w][0][lane];
        sut += L.part[slot][w][1][lane];
      }
      if (c < m) {
        float4 o;
        o.x = silu_mul(sgt[0], sut[0]);
        o.y = silu_mul(sgt[1], sut[1]);
        o.z = silu_mul(sgt[2], sut[2]);
        o.w = silu_mul(sgt[3], sut[3]);
        *reinterpret_cast<float4*>(a.a_buf + (int64_t)pair * I + i0 + 4 * g) = o;
      }
      if (lane == 0) {
        L.arrive[slot] = 0;
        __hip_atomic_store(&L.slot_tile[slot], lt + kSlots, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    if (more && !same) {
      switch_expert((t + 1) / tpe);
      if constexpr (kPipe) tile_w_load(a, e, ((t + 1) % tpe) * kTileRows, w0, n, 0, A);
    }
  }
}

// Workgroups [0, Gm) take the matrix-core tiles (split evenly), the others the vector units of
// the remaining experts (cost-weighted); Gm follows the two parts' costs, a tile counting
// kTileCost units.  One launch, so both parts stream at once and share one ramp and tail.
template <int FMT, int NS, int UPG, int WMAX>
__global__ __launch_bounds__(kMfmaThreads) void gateup_mix_kernel(FfnArgs a) {
  constexpr int NWV = kMfmaThreads / kWave;
  __shared__ MfmaLds<NWV> L;
  __shared__ uint32_t bits_v[NWV][kBitmapWords];
  __shared__ int base_v[NWV][kBitmapWords];
  __shared__ int SEL[kMaxPairs];
  const int wave = threadIdx.x / kWave;
  const int n_pairs = a.M * a.S;
  int* cnt = L.q.cnt[wave];
  WaveQueue Q, Qm, Qv;
  tokens_queue<NWV>(a, Q, L.q.bits[wave], L.q.base[wave], SEL);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  class_queue<true>(Q, cnt, L.bits_m[wave], L.base_m[wave], n_pairs, a.n_experts, Qm);
  class_queue<false>(Q, cnt, bits_v[wave], base_v[wave], n_pairs, a.n_experts, Qv);
  WaveBalance Bv;
  wave_balance_build(Bv, Qv, cnt, a.I, kUnitCost, kPairCost);
  const int64_t n_tiles = (int64_t)Qm.n_active * (a.I / kTileRows);
  const int G = gridDim.x;
  const int Gm = role_split(n_tiles * kTileCost, Bv.total, G);
  if ((int)blockIdx.x < Gm) {
    gateup_tiles<FMT, WMAX>(a, L, Qm, (int)(n_tiles * blockIdx.x / Gm),
                            (int)(n_tiles * (blockIdx.x + 1) / Gm));
  } else {
    constexpr int kAlign = UPG == 2 ? ~1 : ~0;
    const int b = blockIdx.x - Gm, Gv = G - Gm;
    const int u0 = wave_balance_unit(Bv, (int64_t)Bv.total * b / Gv) & kAlign;
    const int u1 = wave_balance_unit(Bv, (int64_t)Bv.total * (b + 1) / Gv) & kAlign;
    gateup_range<FMT, NS, UPG, true, false, false>(a, Qv, &L.q.next, u0, u1, nullptr, nullptr);
  }
}

// ---- down projection

// The expert's a in LDS as bf16 pairs (hi, lo) with hi = bf16(a), lo = bf16(a - hi): a is held
// to within 2^-18 of its fp32 value (the vector path multiplies the fp32 value), and the MFMA
// multiplies both parts exactly and accumulates in fp32.  Layout [piece][column] of 8 values
// (piece P: reduction positions 8P..8P+7), so the 16 lanes of one lane group read 256
// contiguous bytes.
constexpr int kDownMaxI = 2048;
struct DownLds {
  QueueLdsT<kMfmaThreads / kWave> q;
  uint32_t bits_m[kMfmaThreads / kWave][kBitmapWords];
  int base_m[kMfmaThreads / kWave][kBitmapWords];
  uint4 ahi[kDownMaxI / 8 * 16];
  uint4 alo[kDownMaxI / 8 * 16];
};

// bf16 bits of a finite fp32 value, nearest even
__device__ __forceinline__ uint32_t bf16_rn(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eight fp32 values as (hi, lo) bf16 pieces; a value that is not finite keeps it in hi alone.
__device__ __forceinline__ void split_bf16x8(float4 f0, float4 f1, uint4& hi, uint4& lo) {
  const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
  uint32_t h[8], l[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t u = __float_as_uint(v[k]);
    const bool fin = (u & 0x7F800000u) != 0x7F800000u;
    h[k] = fin ? bf16_rn(v[k]) : ((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    const float r = v[k] - __uint_as_float(h[k] << 16);
    l[k] = fin ? bf16_rn(r) : 0u;
  }
  hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                  h[6] | (h[7] << 16));
  lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                  l[6] | (l[7] << 16));
}

// One wave's weights of one down tile: 16 rows h0.. of W2 of expert e (lane row c), NWIN
// windows of 128 values (lane group g: 32 of them, one E8M0 scale block), and the rows' scale
// bytes (I / 32 per row).
template <int NW>
struct DownTile {
  uint4 w[NW];
  uint32_t s[NW];  // window w's four scale bytes (lane group g: byte g)
};

// Windows [W0, W0 + NW) of a tile of NWIN windows.
template <int NWIN, int W0, int NW>
__device__ __forceinline__ void down_tile_load(const FfnArgs& a, int e, int h0,
                                               DownTile<NW>& T) {
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15, g = lane >> 4;
  const int H = a.H, I = NWIN * kWinVals;
  const int rb = I / 2;
  const int ebytes = H * rb, sbytes = H * (I >> 5);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.w2s)) + (int64_t)e * sbytes,
      (short)0, sbytes, kRsrcWord3);
  if constexpr (NWIN % 4 == 0 && W0 % 4 == 0 && NW % 4 == 0) {  // whole 16-byte scale blocks
#pragma unroll
    for (int k = 0; k < NW / 4; ++k) {
      const u32x4 b =
          __builtin_amdgcn_raw_buffer_load_b128(rs, (h0 + c) * (I >> 5), 4 * W0 + 16 * k, 0);
      T.s[4 * k] = b.x;
      T.s[4 * k + 1] = b.y;
      T.s[4 * k + 2] = b.z;
      T.s[4 * k + 3] = b.w;
    }
  } else {
#pragma unroll
    for (int w = 0; w < NW; ++w)
      T.s[w] = __builtin_amdgcn_raw_buffer_load_b32(rs, (h0 + c) * (I >> 5), 4 * (W0 + w), 0);
  }
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w2) + (int64_t)e * ebytes, (short)0, ebytes, kRsrcWord3);
  const int v = (h0 + c) * rb + 16 * g;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const u32x4 q = buf_load16(rw, v, 64 * (W0 + w));
    T.w[w] = make_uint4(q.x, q.y, q.z, q.w);
  }
}

// The product of windows [W0, W0 + NW) with the expert's a from LDS, added into d.
template <int W0, int NW>
__device__ __forceinline__ void down_tile_mma(const DownLds& L, const DownTile<NW>& T,
                                              f32x4& d) {
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float sc = e8m0_to_f32((T.s[w] >> (8 * g)) & 0xFFu);
    const uint32_t w4[4] = {T.w[w].x, T.w[w].y, T.w[w].z, T.w[w].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = (16 * (W0 + w) + 4 * g + j) * 16 + c;
      const uint4 bh = L.ahi[idx], bl = L.alo[idx];
      const bf16x8 A = fp4x8_scaled(w4[j], sc);
      d = mfma(A, as_bf16x8(bh.x, bh.y, bh.z, bh.w), d);
      d = mfma(A, as_bf16x8(bl.x, bl.y, bl.z, bl.w), d);
    }
    // keeps the scheduler from hoisting every window's LDS reads ahead of the products, which
    // held them all in registers at once
    __builtin_amdgcn_sched_barrier(0);
  }
}

// o of the tile's 16 rows from h0 (columns < m; lane: rows 4g..4g+3 of column c).
__device__ __forceinline__ void down_tile_store(const FfnArgs& a, const f32x4& d, int h0,
                                                int pair, int m) {
  const int lane = threadIdx.x % kWave;
  const int c = lane & 15, g = lane >> 4;
  if (c < m) {
    *reinterpret_cast<float4*>(a.o_buf + (int64_t)pair * a.H + h0 + 4 * g) =
        make_float4(d[0], d[1], d[2], d[3]);
  }
}

// Down projection of the tiles [t0, t1) of the experts with 2..16 pairs (queue Qm; MXFP4,
// intermediate NWIN * 128), by the whole workgroup.  A tile is 16 rows of W2 over the whole
// intermediate axis; the workgroup's waves take its tiles in turn, expert by expert: the
// expert's a sits in LDS for all of them, so a wave needs no partner and keeps the next tile's
// loads in flight while it multiplies the current one.
template <int NWIN>
__device__ __forceinline__ void down_tiles(const FfnArgs& a, DownLds& L, const WaveQueue& Qm,
                                           int t0, int t1) {
  constexpr int NWV = kMfmaThreads / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int I = NWIN * kWinVals, H = a.H;
  const int tpe = H / kTileRows;
  const int c = lane & 15;
  for (int t = t0; t < t1;) {
    const int q = t / tpe;
    const int end = min(t1, (q + 1) * tpe);
    const int e = wave_queue_expert(Qm, q);
    uint64_t pm[kPairRegs];
    wave_queue_pairs(Qm, q, pm);
    int m = 0;
#pragma unroll
    for (int k = 0; k < kPairRegs; ++k) m += __popcll(pm[k]);
    const int pair = nth_pair(pm, c < m ? c : m - 1);  // column c (thread's column: c too)
    // the expert's a into LDS (every thread fills column c of its pieces)
    __syncthreads();
    for (int idx = threadIdx.x; idx < I / 8 * 16; idx += kMfmaThreads) {
      uint4 hi = make_uint4(0u, 0u, 0u, 0u), lo = hi;
      if (c < m) {
        const float4* src = reinterpret_cast<const float4*>(a.a_buf + (int64_t)pair * I +
                                                            8 * (idx >> 4));
        split_bf16x8(src[0], src[1], hi, lo);
      }
      L.ahi[idx] = hi;
      L.alo[idx] = lo;
    }
    __syncthreads();
    // this wave's tiles t + wave, t + wave + NWV, ... of the expert.  Up to 12 windows a
    // tile's loads fit twice in the registers: the next tile's are in flight while the current
    // one is multiplied.  Past that the tile goes in two halves: the second half's loads are in
    // flight while the first half is multiplied, and the next tile's first half while the
    // second half is.
    constexpr int CH = NWIN > 12 ? 2 : 1;
    constexpr int CW = NWIN / CH;
    int tt = t + wave;
    if constexpr (CH == 1) {
      DownTile<CW> A, B;
      if (tt < end) down_tile_load<NWIN, 0, CW>(a, e, (tt % tpe) * kTileRows, A);
      while (tt < end) {
        if (tt + NWV < end) down_tile_load<NWIN, 0, CW>(a, e, ((tt + NWV) % tpe) * kTileRows, B);
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        down_tile_mma<0, CW>(L, A, d);
        down_tile_store(a, d, (tt % tpe) * kTileRows, pair, m);
        tt += NWV;
        if (tt >= end) break;
        if (tt + NWV < end) down_tile_load<NWIN, 0, CW>(a, e, ((tt + NWV) % tpe) * kTileRows, A);
        d = f32x4{0.f, 0.f, 0.f, 0.f};
        down_tile_mma<0, CW>(L, B, d);
        down_tile_store(a, d, (tt % tpe) * kTileRows, pair, m);
        tt += NWV;
      }
    } else {
      DownTile<CW> A, B;
      if (tt < end) down_tile_load<NWIN, 0, CW>(a, e, (tt % tpe) * kTileRows, A);
      for (; tt < end; tt += NWV) {
        const int h0 = (tt % tpe) * kTileRows;
        down_tile_load<NWIN, CW, CW>(a, e, h0, B);
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        down_tile_mma<0, CW>(L, A, d);
        if (tt + NWV < end) down_tile_load<NWIN, 0, CW>(a, e, ((tt + NWV) % tpe) * kTileRows, A);
        down_tile_mma<CW, CW>(L, B, d);
        down_tile_store(a, d, h0, pair, m);
      }
    }
    t = end;
  }
}

// Workgroups [0, Gm) take the matrix-core down tiles, the others the vector down units of the
// remaining experts (FLAT: the flattened-row body, else the row-chunk body), split as in
// gateup_mix_kernel.  Costs in quarters of a vector pass over 8 rows.  The kernel runs at the
// tiles' two waves per SIMD, so at I = 2048 (one 16-byte chunk per lane and row) the row-chunk
// body takes 16 rows per unit, which its registers then allow: twice the bytes in flight per
// wave (1T MXFP4, 16 tokens: 457-459 -> 442-444 us per layer).
template <int NWIN, bool FLAT>
__global__ __launch_bounds__(kMfmaThreads) void down_mix_kernel(FfnArgs a) {
  constexpr int NWV = kMfmaThreads / kWave;
  constexpr int kRows = (!FLAT && NWIN == 16) ? 16 : 8;
  __shared__ DownLds L;
  __shared__ uint32_t bits_v[NWV][kBitmapWords];
  __shared__ int base_v[NWV][kBitmapWords];
  const int wave = threadIdx.x / kWave;
  const int n_pairs = a.M * a.S;
  int* cnt = L.q.cnt[wave];
  WaveQueue Q, Qm, Qv;
  wave_queue_build(Q, L.q.bits[wave], L.q.base[wave], a.ids, n_pairs, a.n_experts);
  if (Q.invalid && blockIdx.x == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
  class_queue<true>(Q, cnt, L.bits_m[wave], L.base_m[wave], n_pairs, a.n_experts, Qm);
  class_queue<false>(Q, cnt, bits_v[wave], base_v[wave], n_pairs, a.n_experts, Qv);
  WaveBalance Bv;
  wave_balance_build(Bv, Qv, cnt, a.H / kRows, kRows / 2 * kUnitCost, kRows / 2 * kPairCost);
  const int64_t n_tiles = (int64_t)Qm.n_active * (a.H / kTileRows);
  const int G = gridDim.x;
  const int Gm = role_split(n_tiles * kDownTileCost, Bv.total, G);
  if ((int)blockIdx.x < Gm) {
    down_tiles<NWIN>(a, L, Qm, (int)(n_tiles * blockIdx.x / Gm),
                     (int)(n_tiles * (blockIdx.x + 1) / Gm));
  } else {
    const int b = blockIdx.x - Gm, Gv = G - Gm;
    const int v0 = wave_balance_unit(Bv, (int64_t)Bv.total * b / Gv);
    const int v1 = wave_balance_unit(Bv, (int64_t)Bv.total * (b + 1) / Gv);
    if (threadIdx.x == 0) L.q.next = v0;
    __syncthreads();
    if constexpr (FLAT) {
      // the vector workgroups hold no matrix-core tiles: their waves' rows of a go in ahi
      static_assert(sizeof(L.ahi) >= NWV * 1536 * sizeof(float), "one a row per wave");
      down_flat_dyn<WFMT_MXFP4, 96, 12, 8>(a, Qv, v1, &L.q.next,
                                           reinterpret_cast<float*>(L.ahi) + wave * 1536);
    } else {
      NoReport rep;
      down_rows_range<WFMT_MXFP4, 1, kRows, true, false, false>(a, Qv, &L.q.next, v0, v1, rep);
    }
  }
}

template <typename K>
hipError_t launch_resident(K kern, int* grid, int tpb, const FfnArgs& a, hipStream_t stream) {
  hipError_t err = resident_grid(kern, grid, tpb);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(*grid), dim3(tpb), 0, stream, a);
  return hipGetLastError();
}

template <int FMT, int NS, int WMAX>
hipError_t launch_gateup_mix(const FfnArgs& a, hipStream_t stream) {
  constexpr int UPG = NS <= (FMT == WFMT_FP8_B128 ? 5 : 3) ? 1 : 2;
  static int grid = 0;
  return launch_resident(gateup_mix_kernel<FMT, NS, UPG, WMAX>, &grid, kMfmaThreads, a, stream);
}

// WMAX: windows of 128 values per wave, ceil(H / 128 / 8), which NS (chunks of 16 bytes per lane
// of a row) bounds: 2NS - 1 or 2NS for MXFP4, NS for FP8; up to 8 (MXFP4) or 5 (FP8), which
// the registers hold.
template <int FMT, int NS>
hipError_t launch_mfma_t(const FfnArgs& a, hipStream_t stream) {
  constexpr int NWV = kMfmaThreads / kWave;
  const int per_wave = (a.H / kWinVals + NWV - 1) / NWV;
  if constexpr (FMT == WFMT_MXFP4) {
    if (per_wave <= 2 * NS - 1) return launch_gateup_mix<FMT, NS, 2 * NS - 1>(a, stream);
    return launch_gateup_mix<FMT, NS, 2 * NS>(a, stream);
  } else {
    if (NS <= 5 && per_wave <= NS) return launch_gateup_mix<FMT, NS, NS>(a, stream);
    return hipErrorNotSupported;
  }
}

template <int NWIN, bool FLAT>
hipError_t launch_down_mix(const FfnArgs& a, hipStream_t stream) {
  static int grid = 0;
  return launch_resident(down_mix_kernel<NWIN, FLAT>, &grid, kMfmaThreads, a, stream);
}

}  // namespace

hipError_t launch_gate_up_mfma(const FfnArgs& a, int wfmt, hipStream_t stream) {
  if (a.M < kMfmaMinTokens || a.H % kWinVals != 0 || a.I % kTileRows != 0) return hipErrorNotSupported;
  const int ns = ffn_chunks_per_lane(wfmt, a.H);
  if (wfmt == WFMT_MXFP4) {
    switch (ns) {
      case 1: return launch_mfma_t<WFMT_MXFP4, 1>(a, stream);
      case 2: return launch_mfma_t<WFMT_MXFP4, 2>(a, stream);
      case 3: return launch_mfma_t<WFMT_MXFP4, 3>(a, stream);
      case 4: return launch_mfma_t<WFMT_MXFP4, 4>(a, stream);
      default: return hipErrorNotSupported;
    }
  }
  if (wfmt == WFMT_FP8_B128) {
    switch (ns) {
      case 1: return launch_mfma_t<WFMT_FP8_B128, 1>(a, stream);
      case 2: return launch_mfma_t<WFMT_FP8_B128, 2>(a, stream);
      case 3: return launch_mfma_t<WFMT_FP8_B128, 3>(a, stream);
      case 4: return launch_mfma_t<WFMT_FP8_B128, 4>(a, stream);
      case 5: return launch_mfma_t<WFMT_FP8_B128, 5>(a, stream);
      default: return hipErrorNotSupported;
    }
  }
  return hipErrorNotSupported;
}


hipError_t launch_down_mfma(const FfnArgs& a, int wfmt, hipStream_t stream) {
  if (a.M < kMfmaMinTokens || wfmt != WFMT_MXFP4 || a.H % kTileRows != 0)
    return hipErrorNotSupported;
  hipError_t err = hipErrorNotSupported;
  switch (a.I) {
    case 256: err = launch_down_mix<2, false>(a, stream); break;
    case 384: err = launch_down_mix<3, false>(a, stream); break;
    case 1536: err = launch_down_mix<12, true>(a, stream); break;
    case 2048: err = launch_down_mix<16, false>(a, stream); break;
    default: return hipErrorNotSupported;
  }
  if (err != hipSuccess) return err;
  return launch_combine(a, stream);
}

}  // namespace moe
