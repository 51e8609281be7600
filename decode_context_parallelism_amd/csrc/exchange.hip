// The DCP exchange around the cross-rank merge, on one rank's side.
//
// "Context Parallel Guide (PCP & DCP)", comm_backend (a2a): every rank sends
// each peer that peer's head slice of its partial output with the LSE packed
// alongside, in one all-to-all, and the combine is done locally; the fp32 LSE
// travels as two 16-bit halves of the bf16 buffer, so the round trip is exact.
// enable_project_before_merge (PBM): the merge is a per-(token, head) scalar
// weighting plus a cross-rank sum and W_V is a per-head linear map, so W_V can
// be applied to each rank's partial before the exchange; the payload then
// carries v_head_dim values per head instead of the 512 latent dims.
//
// Message layout (bf16 elements): [W peers][T tokens][H/W heads][D + 8], with
// the D output values first, the LSE's low and high 16 bits in slots D and
// D + 1, and zeros in the remaining six (a 16-byte aligned row).  The
// all-to-all itself (send block p of rank r becomes receive block r of rank p)
// is a collective and is not part of this library.
#include "common.h"
#include "launch.h"

namespace dcpmla {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ inline float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ inline uint32_t pack2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

}  // namespace

// One wave per (token, head) source row; lanes below D/8 move 8 values each.
__global__ void __launch_bounds__(256) a2a_pack_kernel(int W, int64_t T, int H, int D,
                                                       const uint4 *__restrict__ o, const float *__restrict__ lse,
                                                       uint16_t *__restrict__ send) {
  const int lane = threadIdx.x & 63;
  const int64_t src = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // t * H + h
  if (src >= T * H) return;
  const int64_t t = src / H;
  const int h = (int)(src - t * H);
  const int Hl = H / W;
  const int p = h / Hl, j = h - p * Hl;
  const int stride = D + 8;
  uint16_t *dst = send + (((int64_t)p * T + t) * Hl + j) * stride;
  if (lane < D / 8) ((uint4 *)dst)[lane] = o[src * (D / 8) + lane];
  if (lane == 0) {
    const uint32_t bits = __float_as_uint(lse[src]);
    ((uint4 *)(dst + D))[0] = make_uint4(bits, 0u, 0u, 0u);   // low half, high half, zeros
  }
}

// One wave per (token, local head) row of this rank's slice: the LSE merge of
// the W received partials, in the order and arithmetic of the rank merge.
__global__ void __launch_bounds__(256) a2a_combine_kernel(int W, int64_t T, int Hl, int D,
                                                          const uint16_t *__restrict__ recv,
                                                          uint4 *__restrict__ out, float *__restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // t * Hl + j
  if (row >= T * Hl) return;
  const int stride = D + 8;
  const int64_t rows = T * Hl;
  auto msg = [&](int r) { return recv + ((int64_t)r * rows + row) * stride; };
  auto lse_of = [&](int r) {
    const uint16_t *m = msg(r) + D;
    return __uint_as_float((uint32_t)m[0] | ((uint32_t)m[1] << 16));
  };
  float mx = kNegInf;
  for (int r = 0; r < W; ++r) mx = fmaxf(mx, lse_of(r));
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float L = kNegInf;
  const bool active = lane < D / 8;
  if (mx > kNegInf) {
    float z = 0.f;
    for (int r = 0; r < W; ++r) {
      const float l = lse_of(r);
      if (!(l > kNegInf)) continue;
      const float w = __builtin_amdgcn_exp2f((l - mx) * kLog2e);
      z += w;
      if (active) {
        const uint4 u = ((const uint4 *)msg(r))[lane];
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += w * bf16_bits_to_f32(wd[k] & 0xFFFFu);
          acc[2 * k + 1] += w * bf16_bits_to_f32(wd[k] >> 16);
        }
      }
    }
    const float inv = 1.f / z;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= inv;
    L = mx + __builtin_amdgcn_logf(z) * kLn2;
  }
  if (active)
    out[row * (D / 8) + lane] = make_uint4(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]),
                                           pack2(acc[4], acc[5]), pack2(acc[6], acc[7]));
  if (lane == 0) lse[row] = L;
}

// PBM projection: out[t, h, n] = sum_k o[t, h, k] * W_V[h][k][n], with W_V
// supplied transposed (wvt[h][n][k]).  One wave per (head, 32 tokens, 32
// output dims): C = W_V^T O^T on v_mfma_f32_32x32x16_bf16, A = 32 rows of
// wvt (lane = output dim), B = 32 token rows of o (lane = token), so each
// lane ends with 16 output dims of one token, four consecutive at a time.
__global__ void __launch_bounds__(256) project_heads_kernel(int64_t T, int H, int DV,
                                                            const uint16_t *__restrict__ o,
                                                            const uint16_t *__restrict__ wvt,
                                                            uint16_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hk = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int64_t t = t0 + l32;
  const bool tok = t < T;
  const uint16_t *orow = o + ((tok ? t : T - 1) * H + h) * (int64_t)kDv;
  const uint32_t keep = tok ? 0xFFFFFFFFu : 0u;
  for (int n0 = wave * 32; n0 < DV; n0 += 4 * 32) {
    const uint16_t *wrow = wvt + ((int64_t)h * DV + n0 + l32) * kDv;
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll 8
    for (int k0 = 0; k0 < kDv; k0 += 16) {
      const uint4 a = *(const uint4 *)(wrow + k0 + 8 * hk);
      uint4 b = *(const uint4 *)(orow + k0 + 8 * hk);
      b.x &= keep; b.y &= keep; b.z &= keep; b.w &= keep;
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    if (tok) {
      uint16_t *dst = out + (t * H + h) * (int64_t)DV + n0;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = 8 * g4 + 4 * hk;
        *(uint2 *)(dst + n) = make_uint2(pack2(acc[4 * g4 + 0], acc[4 * g4 + 1]),
                                         pack2(acc[4 * g4 + 2], acc[4 * g4 + 3]));
      }
    }
  }
}

hipError_t launch_a2a_pack(int world, int64_t tokens, int heads, int dim, const void *out_rank,
                           const float *lse_rank, void *send, hipStream_t stream) {
  const int64_t rows = tokens * heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(a2a_pack_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, world,
                     tokens, heads, dim, (const uint4 *)out_rank, lse_rank, (uint16_t *)send);
  return hipGetLastError();
}

hipError_t launch_a2a_combine(int world, int64_t tokens, int heads_local, int dim, const void *recv,
                              void *out, float *lse, hipStream_t stream) {
  const int64_t rows = tokens * heads_local;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(a2a_combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, world,
                     tokens, heads_local, dim, (const uint16_t *)recv, (uint4 *)out, lse);
  return hipGetLastError();
}

hipError_t launch_project_heads(int64_t tokens, int heads, int dv, const void *o, const void *wvt,
                                void *out, hipStream_t stream) {
  if (tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(project_heads_kernel, dim3((unsigned)((tokens + 31) / 32), heads), dim3(256), 0,
                     stream, tokens, heads, dv, (const uint16_t *)o, (const uint16_t *)wvt,
                     (uint16_t *)out);
  return hipGetLastError();
}

}  // namespace dcpmla
