// Segmented split-KV MLA attention for one DCP rank (gfx950, BF16 MFMA).
//
// What it computes ("[ROCm][MLA][DCP] Support causal multi-token
// verification", vLLM PR #51705, "Implementation" items 1-3; the shared
// latent head from "Context Parallel Guide (PCP & DCP)", opening of the DCP
// guide): for every verify row (b, i) and gathered head h, softmax attention
// of q[b,i,h,0:576] over the rank-local latent rows 0 .. len(b,i)-1 of
// sequence b, keys = all 576 dims, values = dims 0..511.  Every head of every
// verify row reads the same latent rows, so M = qlen * H head-rows share one
// pass over the sequence's KV; the verify rows differ only in how many of the
// leading rank-local tokens they may see (the window of a row is a prefix of
// the rank-local token list).
//
// Work decomposition (persistent, stream-K style).  A unit is one 32-token
// stage of one (sequence b, tile of 128 head-rows).  Units are ordered
// sequence-major, tile, stage; workgroup w of G takes units
// [w*U/G, (w+1)*U/G).  A (b, tile) whose stages all fall inside one workgroup
// is finished here (BF16 output + natural-log LSE); otherwise each workgroup
// writes an unreduced partial (normalised fp32 output + base-2 LSE) to one of
// its two workspace slots and the segment merge finishes the row.  The grid
// depends only on the device, the unit count only on device metadata, so the
// launch is capture-stable.
//
// Inside a workgroup: 4 waves x 32 head-rows.  Each wave keeps its 32 query
// rows (32 x 576 BF16) in registers as the B operand of S^T = K Q^T
// (v_mfma_f32_32x32x16_bf16, A = K tile from LDS), so a lane's scores all
// belong to one head-row and the online softmax needs one cross-half swap.
// The probabilities P^T stay in registers as the B operand of
// O^T = V^T P^T; the 512 x 32 output accumulator lives in 16 MFMA
// accumulators (256 AGPRs).  KV stages are double-buffered in LDS in the
// cache's own element format (FP8 bytes or BF16), K as [d/16][token][16] and
// V^T as [token/16][half][d][8] (transposed in registers while staging), and
// are widened to BF16 in registers right before each MFMA: E4M3 -> BF16 is
// exact, so the kv scale folds into the score scale and the output.
#include "common.h"
#include "launch.h"

namespace dcpmla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // keep a stale running max while 2^(s - m) <= 2^8

constexpr int kKElems = (kDqk / 16) * kStageTokens * 16;   // K part of one stage
constexpr int kVElems = 2 * 2 * kDv * 8;                   // V^T part of one stage
constexpr int kStageElems = kKElems + kVElems;

struct AttnArgs {
  const uint16_t *q;         // [B, qlen, H, 576] bf16 bits
  const uint8_t *pool;       // [num_pages * P, 576] cache elements
  const int32_t *row_len;    // [B*qlen]
  const int32_t *page_table; // [B*qlen, max_local_pages]
  const int32_t *work;
  float *ws_o;               // [G][2][128][512]
  float *ws_lse2;            // [G][2][128]
  uint16_t *out;             // [B, qlen, H, 512] bf16 bits
  float *lse;                // [B, qlen, H]
  int32_t *err;
  int64_t num_pages;
  int B, qlen, H, M, n_mt, page_shift, max_local_pages;
  float score_scale2;        // softmax_scale * kv_scale * log2(e)
  float out_scale;           // kv_scale
};

// token (within a 32-token stage) held by register r of a 32x32 accumulator
// in lane half h: rows 8*(r/4) + 4*h + r%4 of the MFMA output tile
__device__ inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int E>
struct Staged;

template <>
struct Staged<1> {
  uint2 v[8];
  uint4 rope;
};

template <>
struct Staged<2> {
  uint4 v[8];
  uint4 rope[2];
};

__device__ inline bf16x8 widen_fp8(uint2 raw) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

template <int E>
__device__ inline bf16x8 lds_operand(const uint8_t *p) {
  if constexpr (E == 1) {
    return widen_fp8(*(const uint2 *)p);
  } else {
    return __builtin_bit_cast(bf16x8, *(const uint4 *)p);
  }
}

// 8x8 transpose of byte elements held as 8 rows of 64 bits
__host__ __device__ inline void transpose8x8_b8(uint64_t r[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t a = r[j], b = r[j + 4];
    r[j] = (a & 0x00000000FFFFFFFFull) | (b << 32);
    r[j + 4] = (a >> 32) | (b & 0xFFFFFFFF00000000ull);
  }
#pragma unroll
  for (int j0 = 0; j0 < 8; j0 += 4) {
#pragma unroll
    for (int j = j0; j < j0 + 2; ++j) {
      const uint64_t a = r[j], b = r[j + 2];
      r[j] = (a & 0x0000FFFF0000FFFFull) | ((b << 16) & 0xFFFF0000FFFF0000ull);
      r[j + 2] = ((a >> 16) & 0x0000FFFF0000FFFFull) | (b & 0xFFFF0000FFFF0000ull);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const uint64_t a = r[j], b = r[j + 1];
    r[j] = (a & 0x00FF00FF00FF00FFull) | ((b << 8) & 0xFF00FF00FF00FF00ull);
    r[j + 1] = ((a >> 8) & 0x00FF00FF00FF00FFull) | (b & 0xFF00FF00FF00FF00ull);
  }
}

// 8x8 transpose of 16-bit elements held as 8 rows of 128 bits (lo, hi words)
__host__ __device__ inline void transpose8x8_b16(uint64_t lo[8], uint64_t hi[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // swap 4x4 blocks
    const uint64_t t = hi[j];
    hi[j] = lo[j + 4];
    lo[j + 4] = t;
  }
#pragma unroll
  for (int j0 = 0; j0 < 8; j0 += 4) {
#pragma unroll
    for (int j = j0; j < j0 + 2; ++j) {
      uint64_t a = lo[j], b = lo[j + 2];
      lo[j] = (a & 0x00000000FFFFFFFFull) | (b << 32);
      lo[j + 2] = (a >> 32) | (b & 0xFFFFFFFF00000000ull);
      a = hi[j];
      b = hi[j + 2];
      hi[j] = (a & 0x00000000FFFFFFFFull) | (b << 32);
      hi[j + 2] = (a >> 32) | (b & 0xFFFFFFFF00000000ull);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    uint64_t a = lo[j], b = lo[j + 1];
    lo[j] = (a & 0x0000FFFF0000FFFFull) | ((b << 16) & 0xFFFF0000FFFF0000ull);
    lo[j + 1] = ((a >> 16) & 0x0000FFFF0000FFFFull) | (b & 0xFFFF0000FFFF0000ull);
    a = hi[j];
    b = hi[j + 1];
    hi[j] = (a & 0x0000FFFF0000FFFFull) | ((b << 16) & 0xFFFF0000FFFF0000ull);
    hi[j + 1] = ((a >> 16) & 0x0000FFFF0000FFFFull) | (b & 0xFFFF0000FFFF0000ull);
  }
}

template <int E>
struct Stager {
  // thread roles while staging one 32-token stage:
  //   wave -> (kb, sh) = 16-token half and lane-half of the V^T layout,
  //   lane -> 8-dim chunk c of the 512 value dims (the same bytes feed K);
  //   threads < 128 also move one 16-dim piece of the 64 rope dims.
  int kb, sh, c, rtok, rpart;
  __device__ Stager(int tid) {
    const int wave = tid >> 6;
    kb = wave >> 1;
    sh = wave & 1;
    c = tid & 63;
    rtok = (tid >> 2) & 31;
    rpart = tid & 3;
  }
  __device__ int token(int j) const { return 16 * kb + 8 * (j >> 2) + 4 * sh + (j & 3); }
};

template <int E>
__device__ inline int64_t row_offset(const AttnArgs &a, const int32_t *pt, int t, int32_t *bad) {
  // element offset of rank-local token t's latent row, or -1 (bad page id)
  const int j = t >> a.page_shift;
  const int32_t pg = pt[j];
  if (pg < 0 || (int64_t)pg >= a.num_pages) {
    *bad = 1;
    return -1;
  }
  return (((int64_t)pg << a.page_shift) + (t & ((1 << a.page_shift) - 1))) * kDqk;
}

template <int E>
__device__ inline void load_stage(const AttnArgs &a, const Stager<E> &sg, const int32_t *pt,
                                  int s, int lmax, int tid, Staged<E> &st, int32_t *bad) {
  // Tokens past the sequence's longest row, and tokens on a bad page, load
  // pool row 0 (always a valid address) and are zeroed, so LDS never holds
  // stale bytes (an FP8 NaN pattern times a zero probability would poison
  // the output).
  const int t0 = s * kStageTokens;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = t0 + sg.token(j);
    const int64_t off = t < lmax ? row_offset<E>(a, pt, t, bad) : -1;
    const int64_t src = off >= 0 ? off : 0;
    const uint32_t keep = off >= 0 ? 0xFFFFFFFFu : 0u;
    if constexpr (E == 1) {
      uint2 v = *(const uint2 *)(a.pool + src + 8 * sg.c);
      v.x &= keep; v.y &= keep;
      st.v[j] = v;
    } else {
      uint4 v = *(const uint4 *)(a.pool + 2 * (src + 8 * sg.c));
      v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
      st.v[j] = v;
    }
  }
  {
    const int t = t0 + sg.rtok;
    const int64_t off = (tid < 128 && t < lmax) ? row_offset<E>(a, pt, t, bad) : -1;
    const int64_t src = off >= 0 ? off : 0;
    const uint32_t keep = off >= 0 ? 0xFFFFFFFFu : 0u;
    if constexpr (E == 1) {
      uint4 v = *(const uint4 *)(a.pool + src + kDv + 16 * sg.rpart);
      v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
      st.rope = v;
    } else {
      const uint4 *p = (const uint4 *)(a.pool + 2 * (src + kDv + 16 * sg.rpart));
      uint4 v0 = p[0], v1 = p[1];
      v0.x &= keep; v0.y &= keep; v0.z &= keep; v0.w &= keep;
      v1.x &= keep; v1.y &= keep; v1.z &= keep; v1.w &= keep;
      st.rope[0] = v0;
      st.rope[1] = v1;
    }
  }
}

template <int E>
__device__ inline void store_stage(uint8_t *sb, const Stager<E> &sg, int tid, const Staged<E> &st) {
  // K: [kk = d/16][token][16 elems]; this thread's chunk is half (c & 1) of kk = c/2
  const int kk = sg.c >> 1;
  const int half = sg.c & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint8_t *dst = sb + (((kk * kStageTokens + sg.token(j)) * 16 + 8 * half) * E);
    if constexpr (E == 1) *(uint2 *)dst = st.v[j];
    else *(uint4 *)dst = st.v[j];
  }
  // V^T: [kb][sh][d][8 tokens in accumulator-row order]
  uint8_t *vt = sb + kKElems * E + (((sg.kb * 2 + sg.sh) * kDv + 8 * sg.c) * 8) * E;
  if constexpr (E == 1) {
    uint64_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (uint64_t)st.v[j].x | ((uint64_t)st.v[j].y << 32);
    transpose8x8_b8(r);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *(uint4 *)(vt + 16 * k) = make_uint4((uint32_t)r[2 * k], (uint32_t)(r[2 * k] >> 32),
                                           (uint32_t)r[2 * k + 1], (uint32_t)(r[2 * k + 1] >> 32));
  } else {
    uint64_t lo[8], hi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo[j] = (uint64_t)st.v[j].x | ((uint64_t)st.v[j].y << 32);
      hi[j] = (uint64_t)st.v[j].z | ((uint64_t)st.v[j].w << 32);
    }
    transpose8x8_b16(lo, hi);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      *(uint4 *)(vt + 16 * k) = make_uint4((uint32_t)lo[k], (uint32_t)(lo[k] >> 32), (uint32_t)hi[k],
                                           (uint32_t)(hi[k] >> 32));
  }
  if (tid < 128) {
    uint8_t *dst = sb + ((((kDv / 16) + sg.rpart) * kStageTokens + sg.rtok) * 16) * E;
    if constexpr (E == 1) {
      *(uint4 *)dst = st.rope;
    } else {
      *(uint4 *)dst = st.rope[0];
      *(uint4 *)(dst + 16) = st.rope[1];
    }
  }
}

template <int E>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attention_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int64_t U = a.work[0];
  if (U == 0) return;
  const int64_t G = effective_groups(gridDim.x, U);
  const int64_t w = blockIdx.x;
  if (w >= G) return;
  const int64_t lo = group_lo(w, U, G);
  const int64_t hi = group_lo(w + 1, U, G);
  const int32_t *unit_base = a.work + work_unit_base_off();
  const Stager<E> sg(tid);
  int32_t bad = 0;

  int slot = 0;
  for (int64_t u = lo; u < hi;) {
    // locate the (sequence, tile) piece that holds unit u
    int blo = 0, bhi = a.B;   // unit_base[blo] <= u < unit_base[bhi]
    while (bhi - blo > 1) {
      const int mid = (blo + bhi) >> 1;
      if ((int64_t)unit_base[mid] <= u) blo = mid; else bhi = mid;
    }
    const int b = blo;
    const int stages = a.work[work_stages_off(a.B) + b];
    const int64_t rem = u - unit_base[b];
    const int mt = (int)(rem / stages);
    const int st0 = (int)(rem - (int64_t)mt * stages);
    const int st1 = (int)min((int64_t)stages, st0 + (hi - u));
    const bool complete = st0 == 0 && st1 == stages;
    const int lmax = a.work[work_lmax_off(a.B) + b];
    const int32_t *pt = a.page_table + (int64_t)a.work[work_lrow_off(a.B) + b] * a.max_local_pages;

    // this lane's head-row and its verify-row window
    const int m = mt * kTileRows + wave * kWaveRows + l32;
    const bool mvalid = m < a.M;
    const int vrow = mvalid ? m / a.H : 0;
    const int rlen = mvalid ? a.row_len[b * a.qlen + vrow] : 0;

    bf16x8 qf[kDqk / 16];
    {
      // rows past M read row M-1 (a valid address) and are zeroed
      const uint16_t *qrow = a.q + ((int64_t)b * a.M + (mvalid ? m : a.M - 1)) * kDqk + 8 * h;
      const uint32_t keep = mvalid ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int kk = 0; kk < kDqk / 16; ++kk) {
        uint4 v = *(const uint4 *)(qrow + 16 * kk);
        v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
        qf[kk] = __builtin_bit_cast(bf16x8, v);
      }
    }

    floatx16 oacc[kDv / 32];
#pragma unroll
    for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    float mrun = kNegInf;
    float lsum = 0.f;    // sum of the BF16 probabilities fed to the PV MFMAs: normalises O
    float lsum_f = 0.f;  // fp32 sum of the same probabilities before rounding: gives the LSE

    Staged<E> st;
    load_stage<E>(a, sg, pt, st0, lmax, tid, st, &bad);
    store_stage<E>(lds, sg, tid, st);
    __syncthreads();

    for (int s = st0; s < st1; ++s) {
      const int cur = (s - st0) & 1;
      const bool more = s + 1 < st1;
      if (more) load_stage<E>(a, sg, pt, s + 1, lmax, tid, st, &bad);
      const uint8_t *sb = lds + cur * (kStageElems * E);

      // S^T[token, row] = K Q^T over 576 dims
      floatx16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < kDqk / 16; ++kk) {
        const bf16x8 kop = lds_operand<E>(sb + ((kk * kStageTokens + l32) * 16 + 8 * h) * E);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[kk], sacc, 0, 0, 0);
      }

      // online softmax in base 2 on this lane's 16 tokens of head-row m
      const int t0 = s * kStageTokens;
      float sv[16];
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool valid = t0 + acc_row(r, h) < rlen;
        sv[r] = valid ? sacc[r] * a.score_scale2 : kNegInf;
        mx = fmaxf(mx, sv[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun, mx);
      const bool need = mnew > mrun + kRescaleSlack;
      if (__any(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
        if (need) mrun = mnew;
        lsum *= alpha;
        lsum_f *= alpha;
        // Rare path.  Each accumulator element is scaled in place (read from
        // its AGPR, multiply, write back) so the 256-element accumulator never
        // has to be copied into VGPRs as a whole; the trailing nops cover the
        // VALU-writes-AGPR -> MFMA-reads-SrcC wait states.
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float t;
            asm volatile(
                "v_accvgpr_read_b32 %0, %1\n\t"
                "s_nop 1\n\t"
                "v_mul_f32 %0, %0, %2\n\t"
                "v_accvgpr_write_b32 %1, %0\n\t"
                "s_nop 2"
                : "=&v"(t), "+a"(oacc[d][r])
                : "v"(alpha));
          }
        }
      }
      bf16x8 pb[2];
      const bool live = mrun > kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = live ? __builtin_amdgcn_exp2f(sv[r] - mrun) : 0.f;
        const __bf16 pr = (__bf16)p;
        pb[r >> 3][r & 7] = pr;
        lsum += (float)pr;
        lsum_f += p;
      }

      // O^T[d, row] += V^T[d, token] P^T[token, row]
#pragma unroll
      for (int d = 0; d < kDv / 32; ++d) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 vop =
              lds_operand<E>(sb + kKElems * E + (((kb * 2 + h) * kDv + 32 * d + l32) * 8) * E);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kb], oacc[d], 0, 0, 0);
        }
      }

      if (more) store_stage<E>(lds + (cur ^ 1) * (kStageElems * E), sg, tid, st);
      __syncthreads();
    }

    // finish the piece
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float ltot_f = lsum_f + __shfl_xor(lsum_f, 32);
    const bool has = ltot > 0.f;
    const float inv = has ? a.out_scale / ltot : 0.f;
    const float lse2 = has ? mrun + __builtin_amdgcn_logf(ltot_f) : kNegInf;
    if (complete) {
      if (mvalid) {
        uint16_t *orow = a.out + ((int64_t)b * a.M + m) * kDv;
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dim = 32 * d + 8 * g4 + 4 * h;
            uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(oacc[d][4 * g4 + 0] * inv)) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(oacc[d][4 * g4 + 1] * inv)) << 16);
            uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(oacc[d][4 * g4 + 2] * inv)) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(oacc[d][4 * g4 + 3] * inv)) << 16);
            *(uint2 *)(orow + dim) = make_uint2(w0, w1);
          }
        }
        if (h == 0) a.lse[(int64_t)b * a.M + m] = has ? lse2 * kLn2 : kNegInf;
      }
    } else {
      const int64_t prow = (w * kSlots + slot) * kTileRows + wave * kWaveRows + l32;
      float *orow = a.ws_o + prow * kDv;
#pragma unroll
      for (int d = 0; d < kDv / 32; ++d) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dim = 32 * d + 8 * g4 + 4 * h;
          *(float4 *)(orow + dim) = make_float4(oacc[d][4 * g4 + 0] * inv, oacc[d][4 * g4 + 1] * inv,
                                                oacc[d][4 * g4 + 2] * inv, oacc[d][4 * g4 + 3] * inv);
        }
      }
      if (h == 0) a.ws_lse2[prow] = lse2;
    }
    u += st1 - st0;
    slot = 1;
  }
  if (bad) atomicOr(a.err, DCPMLA_ERR_PAGE_RANGE);
}

}  // namespace

hipError_t launch_partial_attention(const dcpmla_geom &g, int groups, const void *q,
                                    const void *kv_pool, float kv_scale, float softmax_scale,
                                    const dcpmla_meta &m, void *workspace, void *out_rank,
                                    float *lse_rank, hipStream_t stream) {
  AttnArgs a;
  a.q = (const uint16_t *)q;
  a.pool = (const uint8_t *)kv_pool;
  a.row_len = m.row_local_len;
  a.page_table = m.page_table;
  a.work = m.work;
  a.ws_o = (float *)workspace;
  a.ws_lse2 = (float *)workspace + ws_o_floats(groups);
  a.out = (uint16_t *)out_rank;
  a.lse = lse_rank;
  a.err = m.err;
  const int P = subpage_size(g.block_size);
  int shift = 0;
  while ((1 << shift) < P) ++shift;
  a.page_shift = shift;
  a.num_pages = g.num_blocks * (g.block_size / P);
  a.B = g.batch;
  a.qlen = g.qlen;
  a.H = g.num_heads;
  a.M = g.qlen * g.num_heads;
  a.n_mt = n_mtiles(g.qlen, g.num_heads);
  a.max_local_pages = g.max_local_pages;
  a.score_scale2 = softmax_scale * kv_scale * 1.44269504088896340736f;
  a.out_scale = kv_scale;
  if (g.kv_dtype == DCPMLA_KV_FP8_E4M3) {
    const size_t shmem = 2 * kStageElems * 1;
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void *)attention_kernel<1>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    hipLaunchKernelGGL(attention_kernel<1>, dim3(groups), dim3(kThreads), shmem, stream, a);
  } else {
    const size_t shmem = 2 * kStageElems * 2;
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void *)attention_kernel<2>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    hipLaunchKernelGGL(attention_kernel<2>, dim3(groups), dim3(kThreads), shmem, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dcpmla
