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
// Inside a workgroup: 4 waves x 32 head-rows, one wave per SIMD.  Each wave
// keeps its 32 query rows (32 x 576 BF16) in registers as the B operand of
// S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A = K tile read from LDS), so a
// lane's scores all belong to one head-row and the online softmax needs one
// cross-half swap.  The probabilities P^T stay in registers as the B operand
// of O^T = V^T P^T; the 512 x 32 output accumulator lives in 16 MFMA
// accumulators (256 AGPRs).
//
// LDS holds each 32-token stage once, as K blocks [d/16][token][16 elements]
// (one padded block per 16 dims).  The QK operand is a plain read of that
// tile; the PV operand V^T (8 tokens of one value dim per lane) is read from
// the same tile with the gfx950 transposing loads ds_read_b64_tr_b8 /
// ds_read_b64_tr_b16, so no transposed copy of V is kept.  The tile is stored
// either as the cache's FP8 bytes (widened to BF16 in registers before each
// MFMA) or already widened to BF16 while staging; E4M3 -> BF16 is exact, so
// the kv scale folds into the score scale and the output.
#include <stdlib.h>

#include <type_traits>

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

constexpr int kKBlocks = kDqk / 16;                            // 36 blocks of 16 dims
// Staging: 8 threads per token of a 32-token stage; thread (token tid / 8,
// lane-in-token c = tid % 8) moves the 8-element pieces c, c + 8, ..., c + 64
// of its token's 576-element row, so its addresses are one base plus
// constant offsets and it needs one page id per stage.
constexpr int kThreadsPerToken = kThreads / kStageTokens;      // 8
constexpr int kUnitsPerThread = kDqk / 8 / kThreadsPerToken;   // 9
static_assert(kThreadsPerToken * kStageTokens == kThreads, "staging split");

// LDS tile of one stage with L-byte elements: 36 blocks of [32 token slots]
// [16 elements].  Every access pattern (QK rows, transposing PV reads,
// staging stores) covers whole 128-byte bank windows, so blocks need no pad.
template <int L>
struct Tile {
  static constexpr int kRow = 16 * L;
  static constexpr int kBlock = kStageTokens * kRow;
  static constexpr int kBytes = kKBlocks * kBlock;
};

// token (within a 32-token stage) held by register r of a 32x32 accumulator
// in lane half h: rows 8*(r/4) + 4*h + r%4 of the MFMA output tile.  The
// same map assigns PV k-slot 8*h + e (e < 8) of token half kb to token
// 16*kb + tau(h, e).
__device__ inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// LDS row slot of stage-token t.  The PV operand of lane half h gathers the
// eight tokens tau(h, 0..7) = {4h..4h+3, 8+4h..8+4h+3} (+16 for the second
// token half); storing those eight rows in consecutive slots 8h..8h+7 makes
// each 16-lane transposing read touch every bank exactly once.  QK reads all
// 32 rows, in any order, so it does not care.
__host__ __device__ inline int tok_slot(int t) {
  return 16 * (t >> 4) + 8 * ((t >> 2) & 1) + 4 * ((t >> 3) & 1) + (t & 3);
}

template <int E>
struct Staged {
  typedef typename std::conditional<E == 1, uint2, uint4>::type Unit;   // 8 elements
  Unit v[kUnitsPerThread];
  uint32_t keep;   // 1: the token is valid, 0: store zeros
};

__device__ inline uint2 masked(uint2 v, bool k) { return k ? v : make_uint2(0, 0); }
__device__ inline uint4 masked(uint4 v, bool k) { return k ? v : make_uint4(0, 0, 0, 0); }

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

typedef short short4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

// QK operand (A = K): lane (token l32, half h) reads elements 8h..8h+7 of
// block kk of its token
template <int L>
struct KOp {
  typedef typename std::conditional<L == 1, uint2, uint4>::type Raw;
};

template <int L>
__device__ inline typename KOp<L>::Raw lds_k(const uint8_t *sb, int kk, int slot, int h) {
  return *(const typename KOp<L>::Raw *)(sb + kk * Tile<L>::kBlock + slot * Tile<L>::kRow + 8 * h * L);
}

__device__ inline bf16x8 widen_k(uint2 raw) { return widen_fp8(raw); }
__device__ inline bf16x8 widen_k(uint4 raw) { return __builtin_bit_cast(bf16x8, raw); }

// PV operand (A = V^T): lane (dim 32*dblk + l32, half h) gets tokens
// 16*kb + tau(h, e), e = 0..7, of that dim, via transposing reads.  Within a
// 16-lane group the lane that loads address j supplies row j of a 16-row
// (tr_b8: 8-byte, tr_b16: 4-element) block; result lane i receives column
// i % (8 / L... ) of the rows the group loaded -- see the per-format maps.
struct VRaw1 { int2v a; };
struct VRaw2 { short4v a, b; };

template <int L>
struct VOp { typedef typename std::conditional<L == 1, VRaw1, VRaw2>::type Raw; };

__device__ inline VRaw1 lds_v1(const uint8_t *sb, int dblk, int kb, int lane) {
  // tr_b8: result lane 8a+b, byte k = byte b of the row loaded by lane a+2k.
  // Loader j = a + 2k reads token 16kb + tau(h, k), dims d0 + 8a .. d0 + 8a + 7.
  const int g = lane >> 4, j = lane & 15;
  const int h = g >> 1;
  const int kblk = 2 * dblk + (g & 1);
  const int k = j >> 1, a = j & 1;
  const int slot = 16 * kb + 8 * h + k;          // tok_slot(16kb + tau(h, k))
  const uint8_t *p = sb + kblk * Tile<1>::kBlock + slot * Tile<1>::kRow + 8 * a;
  VRaw1 r;
  r.a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) int2v *)(lds_char *)(size_t)p);
  return r;
}

__device__ inline VRaw2 lds_v2(const uint8_t *sb, int dblk, int kb, int lane) {
  // tr_b16: result lane 4a+b, element k = element b of the row loaded by lane
  // a+4k.  Loader j = a + 4k reads token 16kb + tau(h, 4r + k), dims
  // d0 + 4a .. d0 + 4a + 3, for the two halves r = 0, 1 of the 8 k-slots.
  const int g = lane >> 4, j = lane & 15;
  const int h = g >> 1;
  const int kblk = 2 * dblk + (g & 1);
  const int k = j >> 2, a = j & 3;
  const uint8_t *base = sb + kblk * Tile<2>::kBlock + 8 * a;
  const int slot0 = 16 * kb + 8 * h + k;         // tok_slot(16kb + tau(h, k)), k < 4
  const int slot1 = slot0 + 4;                   // tok_slot(16kb + tau(h, 4 + k))
  VRaw2 r;
  r.a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v *)(lds_char *)(size_t)(base + slot0 * Tile<2>::kRow));
  r.b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v *)(lds_char *)(size_t)(base + slot1 * Tile<2>::kRow));
  return r;
}

template <int L>
__device__ inline typename VOp<L>::Raw lds_v(const uint8_t *sb, int dblk, int kb, int lane) {
  if constexpr (L == 1) return lds_v1(sb, dblk, kb, lane);
  else return lds_v2(sb, dblk, kb, lane);
}

__device__ inline bf16x8 widen_v(VRaw1 r) {
  return widen_fp8(make_uint2((uint32_t)r.a[0], (uint32_t)r.a[1]));
}
__device__ inline bf16x8 widen_v(VRaw2 r) {
  // whole-vector reinterpretation (element-wise short -> __bf16 casts into a
  // vector are miscompiled to zeros by this toolchain)
  const uint2 lo = __builtin_bit_cast(uint2, r.a);
  const uint2 hi = __builtin_bit_cast(uint2, r.b);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// ---------------------------------------------------------------- staging

// Issue the global loads of stage s for this thread's token.  A token past
// the longest row, or on a page outside the pool, loads pool row 0 (a valid
// address) and is marked for zeroing, so the LDS tile never holds stale
// bytes (an FP8 NaN pattern times a zero probability would poison the
// output).  Consecutive lanes read consecutive 8-element pieces of a row.
template <int E>
__device__ inline void load_stage(const AttnArgs &a, int32_t page, int s, int lmax, int tid,
                                  Staged<E> &st, int32_t *bad) {
  const int t = s * kStageTokens + tid / kThreadsPerToken;
  const bool in_seq = t < lmax;
  const bool ok = page >= 0 && (int64_t)page < a.num_pages;
  *bad |= (in_seq && !ok) ? 1 : 0;
  const bool valid = in_seq && ok;
  const int64_t row = valid ? ((int64_t)page << a.page_shift) + (t & ((1 << a.page_shift) - 1)) : 0;
  typedef typename Staged<E>::Unit Unit;
  const Unit *src = (const Unit *)(a.pool + (row * kDqk + 8 * (tid % kThreadsPerToken)) * E);
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) st.v[i] = src[i * kThreadsPerToken];
  st.keep = valid ? 1u : 0u;
}

// Write the staged pieces into the LDS tile (widening FP8 to BF16 when L = 2).
// Piece p = c + 8i lands in block p / 2, half p % 2, row token.
template <int E, int L>
__device__ inline void store_stage(uint8_t *sb, int tid, const Staged<E> &st) {
  const int tok = tid / kThreadsPerToken;
  const int c = tid % kThreadsPerToken;
  uint8_t *base = sb + (c >> 1) * Tile<L>::kBlock + tok_slot(tok) * Tile<L>::kRow + 8 * (c & 1) * L;
  const bool keep = st.keep != 0;
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    uint8_t *dst = base + 4 * i * Tile<L>::kBlock;
    const auto v = masked(st.v[i], keep);
    if constexpr (L == 1) {
      *(uint2 *)dst = v;
    } else if constexpr (E == 1) {
      *(uint4 *)dst = __builtin_bit_cast(uint4, widen_fp8(v));
    } else {
      *(uint4 *)dst = v;
    }
  }
}

// Page id of this thread's token of stage s (branch-free: a token past the
// longest row reads slot 0, present whenever the sequence has a token).
__device__ inline int32_t fetch_page(const AttnArgs &a, const int32_t *pt, int s, int lmax, int tid) {
  const int t = s * kStageTokens + tid / kThreadsPerToken;
  return pt[t < lmax ? (t >> a.page_shift) : 0];
}

template <int E, int L>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attention_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];   // two stage tiles
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int kslot = tok_slot(l32);   // LDS slot of the stage token in this lane's score row
  const int64_t U = a.work[0];
  if (U == 0) return;
  const int64_t G = effective_groups(gridDim.x, U);
  const int64_t w = blockIdx.x;
  if (w >= G) return;
  const int64_t lo = group_lo(w, U, G);
  const int64_t hi = group_lo(w + 1, U, G);
  const int32_t *unit_base = a.work + work_unit_base_off();
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

    // page id of this thread's token in the first stage
    int32_t page = fetch_page(a, pt, st0, lmax, tid);

    bf16x8 qf[kKBlocks];
    {
      // rows past M read row M-1 (a valid address) and are zeroed
      const uint16_t *qrow = a.q + ((int64_t)b * a.M + (mvalid ? m : a.M - 1)) * kDqk + 8 * h;
      const uint32_t keep = mvalid ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int kk = 0; kk < kKBlocks; ++kk) {
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
    load_stage<E>(a, page, st0, lmax, tid, st, &bad);
    if (st0 + 1 < st1) page = fetch_page(a, pt, st0 + 1, lmax, tid);
    store_stage<E, L>(lds, tid, st);
    __syncthreads();

    for (int s = st0; s < st1; ++s) {
      const int cur = (s - st0) & 1;
      const bool more = s + 1 < st1;
      if (more) load_stage<E>(a, page, s + 1, lmax, tid, st, &bad);
      if (s + 2 < st1) page = fetch_page(a, pt, s + 2, lmax, tid);
      const uint8_t *sb = lds + cur * Tile<L>::kBytes;

      // S^T[token, row] = K Q^T over 576 dims; operands prefetched two ahead
      floatx16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      {
        typename KOp<L>::Raw kr[2];
        kr[0] = lds_k<L>(sb, 0, kslot, h);
        kr[1] = lds_k<L>(sb, 1, kslot, h);
#pragma unroll
        for (int kk = 0; kk < kKBlocks; ++kk) {
          const bf16x8 kop = widen_k(kr[kk & 1]);
          if (kk + 2 < kKBlocks) kr[kk & 1] = lds_k<L>(sb, kk + 2, kslot, h);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[kk], sacc, 0, 0, 0);
        }
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
      const float alpha = need ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
      // a row that had no visible token yet (mrun = -inf) has O = 0: only rows
      // with earlier mass need their accumulator rescaled
      const bool scale_o = need && mrun > kNegInf;
      if (need) mrun = mnew;
      lsum *= alpha;
      lsum_f *= alpha;
      if (__any(scale_o)) {
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

      // O^T[d, row] += V^T[d, token] P^T[token, row]; operands prefetched two ahead
      {
        typename VOp<L>::Raw vr[2];
        vr[0] = lds_v<L>(sb, 0, 0, lane);
        vr[1] = lds_v<L>(sb, 0, 1, lane);
#pragma unroll
        for (int i = 0; i < kDv / 16; ++i) {
          const int d = i >> 1, kb = i & 1;
          const bf16x8 vop = widen_v(vr[i & 1]);
          if (i + 2 < kDv / 16) vr[i & 1] = lds_v<L>(sb, (i + 2) >> 1, (i + 2) & 1, lane);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kb], oacc[d], 0, 0, 0);
        }
      }

      if (more) store_stage<E, L>(lds + (cur ^ 1) * Tile<L>::kBytes, tid, st);
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
  const size_t extra = 0;
  if (g.kv_dtype == DCPMLA_KV_FP8_E4M3) {
    // FP8 cache: the LDS tile keeps FP8 bytes (widened per operand) unless
    // DCPMLA_LDS_BF16=1 asks for widening once while staging
    static const bool widen_at_stage = getenv("DCPMLA_LDS_BF16") && atoi(getenv("DCPMLA_LDS_BF16")) == 1;
    if (widen_at_stage) {
      const size_t shmem = 2 * Tile<2>::kBytes + extra;
      static bool attr_set = false;
      if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)attention_kernel<1, 2>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess) return e;
        attr_set = true;
      }
      hipLaunchKernelGGL((attention_kernel<1, 2>), dim3(groups), dim3(kThreads), shmem, stream, a);
    } else {
      const size_t shmem = 2 * Tile<1>::kBytes + extra;
      static bool attr_set = false;
      if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)attention_kernel<1, 1>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess) return e;
        attr_set = true;
      }
      hipLaunchKernelGGL((attention_kernel<1, 1>), dim3(groups), dim3(kThreads), shmem, stream, a);
    }
  } else {
    const size_t shmem = 2 * Tile<2>::kBytes + extra;
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void *)attention_kernel<2, 2>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    hipLaunchKernelGGL((attention_kernel<2, 2>), dim3(groups), dim3(kThreads), shmem, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dcpmla
