// Offline weight packing on the GPU: MXFP4 (E2M1 + E8M0 per 32 along K) and FP8 E4M3FN with
// fp32 scales per 128x128 block.  molayo1419.me, "Xiaomi가 어떻게 1조 개의 파라미터를 가진
// 모델에서 초당 1,000 토큰을 달성했는가", section 2 ("MXFP4 with QAT"): 32 values share one
// exponent as the MX specification defines.  Rounding is nearest-even on exact scaled values,
// so the packed bytes are identical to the CPU reference's.
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

// Magnitude t >= 0 (exact fp32) -> E2M1 magnitude code, nearest even, saturating at 6.
// Grid 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); ties (.25, .75, 1.25, 1.75, 2.5, 3.5, 5) go to
// the even code.
__device__ __forceinline__ uint32_t e2m1_rne(float t) {
  if (t <= 0.25f) return 0;
  if (t < 0.75f) return 1;
  if (t <= 1.25f) return 2;
  if (t < 1.75f) return 3;
  if (t <= 2.5f) return 4;
  if (t < 3.5f) return 5;
  if (t <= 5.0f) return 6;
  return 7;
}

// One thread per 32-element block of a row.
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const float* __restrict__ w,
                                                          int64_t rows, int64_t cols,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ s,
                                                          int32_t* nonfinite) {
  const int64_t nblk = cols / 32;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= rows * nblk) return;
  const int64_t r = b / nblk, kb = b % nblk;
  const float4* src = reinterpret_cast<const float4*>(w + r * cols + kb * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f = src[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  int bad = 0;
  uint32_t amax_bits = 0;  // |v| compared as unsigned bit patterns (exact for finite values)
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) ++bad;
    else if (a > amax_bits) amax_bits = a;
  }
  uint4 out = make_uint4(0, 0, 0, 0);
  uint8_t scale;
  if (bad) {
    if (nonfinite) atomicAdd(nonfinite, bad);
    scale = 0xFF;
  } else {
    // floor(log2(amax)) = biased exponent - 127 for normals; subnormals clamp below anyway.
    int X = (amax_bits == 0) ? -127 : (int)(amax_bits >> 23) - 127 - 2;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    scale = (uint8_t)(X + 127);
    // 2^-X as fp32 (X in [-127, 125] here): normal unless X = 127, never reached from fp32.
    const float inv = __uint_as_float((uint32_t)(127 - X) << 23);
    uint32_t words[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t bits = __float_as_uint(v[i]);
      const float t = __uint_as_float(bits & 0x7FFFFFFFu) * inv;  // exact power-of-two scaling
      const uint32_t code = e2m1_rne(t) | ((bits >> 28) & 8u);
      words[i / 8] |= code << (4 * (i % 8));
    }
    out = make_uint4(words[0], words[1], words[2], words[3]);
  }
  reinterpret_cast<uint4*>(q + r * (cols / 2) + kb * 16)[0] = out;
  s[r * nblk + kb] = scale;
}

// One workgroup per 128x128 block: amax, scale = fp32(amax/448), codes of fp32(v/scale).
// Blocks tile the matrix from its origin; the last block along a side that is not a multiple
// of 128 covers the remaining rows / columns only (cols % 16 == 0, so a thread's valid part of
// its 64-column half is whole 16-column groups).  Values outside the matrix read as 0, which
// changes neither the block maximum nor any code, and are never stored.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const float* __restrict__ w,
                                                        int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s,
                                                        int32_t* nonfinite) {
  const int64_t bcs = (cols + 127) / 128;
  const int64_t br = blockIdx.x / bcs, bc = blockIdx.x % bcs;
  const int tid = threadIdx.x;
  // thread -> (row within block = tid/2, 64-column half = tid%2)
  const int rr = tid >> 1, half = tid & 1;
  const int64_t row = br * 128 + rr, col0 = bc * 128 + half * 64;
  // valid columns of this thread's half: a multiple of 16 in [0, 64]
  int64_t nv = row < rows ? cols - col0 : 0;
  nv = nv < 0 ? 0 : (nv > 64 ? 64 : nv);
  const float* src = w + row * cols + col0;
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (4 * i < nv) f = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  int bad = 0;
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) ++bad;
    else if (a > amax_bits) amax_bits = a;
  }
  __shared__ uint32_t red_amax[256 / kWave];
  __shared__ int red_bad[256 / kWave];
  // wave reduction of (max, count)
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t oa = __shfl_xor(amax_bits, o, kWave);
    amax_bits = oa > amax_bits ? oa : amax_bits;
    bad += __shfl_xor(bad, o, kWave);
  }
  if ((tid % kWave) == 0) { red_amax[tid / kWave] = amax_bits; red_bad[tid / kWave] = bad; }
  __syncthreads();
  uint32_t amax = 0;
  int nbad = 0;
#pragma unroll
  for (int i = 0; i < 256 / kWave; ++i) {
    amax = red_amax[i] > amax ? red_amax[i] : amax;
    nbad += red_bad[i];
  }
  uint8_t* dst = q + row * cols + col0;
  if (nbad) {
    if (tid == 0) {
      if (nonfinite) atomicAdd(nonfinite, nbad);
      s[br * bcs + bc] = __builtin_nanf("");
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (16 * i < nv)
        reinterpret_cast<uint4*>(dst)[i] = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu,
                                                      0x7F7F7F7Fu);
    return;
  }
  const float sc = (amax == 0) ? 1.0f : __fdiv_rn(__uint_as_float(amax), 448.0f);
  if (tid == 0) s[br * bcs + bc] = sc;
  uint32_t words[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) words[i] = 0;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const float t = __fdiv_rn(v[i], sc);
    const uint32_t bits = __float_as_uint(t);
    const uint32_t code = e4m3_rne(__uint_as_float(bits & 0x7FFFFFFFu)) | ((bits >> 24) & 0x80u);
    words[i / 4] |= code << (8 * (i % 4));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (16 * i < nv)
      reinterpret_cast<uint4*>(dst)[i] =
          make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
}

}  // namespace

hipError_t launch_quant_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* s, int32_t* nonfinite, hipStream_t stream) {
  const int64_t blocks = rows * (cols / 32);
  const int64_t grid = (blocks + 255) / 256;
  hipLaunchKernelGGL(quant_mxfp4_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w, rows,
                     cols, q, s, nonfinite);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s,
                            int32_t* nonfinite, hipStream_t stream) {
  const int64_t grid = ((rows + 127) / 128) * ((cols + 127) / 128);
  hipLaunchKernelGGL(quant_fp8_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w, rows,
                     cols, q, s, nonfinite);
  return hipGetLastError();
}

}  // namespace moe
