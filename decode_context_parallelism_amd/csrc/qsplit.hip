// Exact two-term E4M3 split of BF16 query rows, for QK on the FP8 matrix
// units against an FP8 cache.
//
// The query is BF16 ("[ROCm][MLA][DCP] Support causal multi-token
// verification": BF16 output from BF16 queries over an FP8 or BF16 latent
// cache; "Context Parallel Guide (PCP & DCP)", "How it works" item 4 for the
// per-tensor-scaled FP8 cache).  Each head-row q is written as
//   q = (hi + lo) * 2^-k,
// k the largest integer with max|q| * 2^k <= 448, hi the E4M3 code nearest to
// x = q * 2^k (ties to even) and lo the code of x - hi.  BF16 carries 8
// significant bits and E4M3 4, so the residual fits one E4M3 code whenever
// |x| >= 2^-2, and then hi + lo = x exactly; below that the split is within
// 2^-10 of x.  K q = (K hi + K lo) * 2^-k then runs as two FP8 products with
// fp32 accumulation, and no FP8 cache element needs widening.
#include "common.h"
#include "launch.h"

namespace dcpmla {

namespace {

typedef short short2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest k with amax * 2^k <= 448 = 1.75 * 2^8 (0 for amax == 0), from the
// bit fields of amax = (1 + f) * 2^(E - 127).
__device__ inline int row_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int extra = 0;
  if (amax < 0x1p-100f) {   // subnormal or close: scale up exactly first
    amax *= 0x1p64f;
    extra = 64;
  }
  const uint32_t bits = __float_as_uint(amax);
  const int E = (int)(bits >> 23);
  const uint32_t mant = bits & 0x7FFFFFu;
  // (1 + f) <= 1.75  <=>  mant <= 0.75 * 2^23
  return (mant <= 0x600000u ? 135 - E : 134 - E) + extra;
}

// Four values -> their E4M3 codes (RNE) in one dword, byte i = value i.
__device__ inline uint32_t to_e4m3x4(float a, float b, float c, float d) {
  short2v w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

__device__ inline void from_e4m3x4(uint32_t codes, float v[4]) {
  const float2v lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, 1.0f, false);
  const float2v hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, 1.0f, true);
  v[0] = lo[0]; v[1] = lo[1]; v[2] = hi[0]; v[3] = hi[1];
}

// 8 BF16 values (one uint4) scaled by 2^k -> 8 hi codes and 8 lo codes.
__device__ inline void split8(uint4 q, int k, uint2 &hi, uint2 &lo) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_ldexpf(bf16_lo(w[i]), k);
    x[2 * i + 1] = __builtin_ldexpf(bf16_hi(w[i]), k);
  }
  const uint32_t h0 = to_e4m3x4(x[0], x[1], x[2], x[3]);
  const uint32_t h1 = to_e4m3x4(x[4], x[5], x[6], x[7]);
  float hv[8];
  from_e4m3x4(h0, hv);
  from_e4m3x4(h1, hv + 4);
  hi = make_uint2(h0, h1);
  lo = make_uint2(to_e4m3x4(x[0] - hv[0], x[1] - hv[1], x[2] - hv[2], x[3] - hv[3]),
                  to_e4m3x4(x[4] - hv[4], x[5] - hv[5], x[6] - hv[6], x[7] - hv[7]));
}

}  // namespace

// One wave per head-row: lanes 0..63 hold dims 8*lane .. +7, lanes 0..7 also
// dims 512 + 8*lane .. +7.  Eight dims d = 8j .. 8j + 7 lie in one 16-byte
// piece of the tiled layout: step t = j / 8, lane half g = j / 4 % 2, half
// j / 2 % 2, byte 8 (j % 2) of the piece.
__global__ void __launch_bounds__(256) split_q_kernel(int64_t rows, const uint4 *__restrict__ q,
                                                      uint8_t *__restrict__ split,
                                                      float *__restrict__ inv_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4 *src = q + row * (kDqk / 8);
  const bool tail = lane < (kDqk - 512) / 8;
  const uint4 v0 = src[lane];
  const uint4 v1 = tail ? src[64 + lane] : make_uint4(0, 0, 0, 0);
  float amax = 0.f;
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const int k = row_exponent(amax);
  // the hi and lo pieces of dims 8j .. 8j + 7
  auto put = [&](int j, uint2 hi, uint2 lo) {
    const int t = j >> 3, g = (j >> 2) & 1, half = (j >> 1) & 1;
    const int64_t off = qsplit_off(row, 4 * t + half, g) + 8 * (j & 1);
    *(uint2 *)(split + off) = hi;
    *(uint2 *)(split + off + 2 * kQSplitChunk) = lo;
  };
  uint2 hi, lo;
  split8(v0, k, hi, lo);
  put(lane, hi, lo);
  if (tail) {
    split8(v1, k, hi, lo);
    put(64 + lane, hi, lo);
  }
  if (lane == 0) inv_scale[row] = __builtin_ldexpf(1.0f, -k);
}

hipError_t launch_split_q(int64_t rows, const void *q, void *split, float *inv_scale, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(split_q_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, rows,
                     (const uint4 *)q, (uint8_t *)split, inv_scale);
  return hipGetLastError();
}

}  // namespace dcpmla
