// Segmented split-KV MLA attention for one DCP rank, BF16 latent cache
// (gfx950, BF16 MFMA).  The FP8-cache kernel is in attention_fp8.hip; both
// share the work walk, staging and argument block of attention_common.h.
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
// sequence-major, tile, stage, and split into G contiguous ranges of equal
// cost, where each (b, tile) item adds a fixed overhead to its stage count
// (its query load and output stores), so a workgroup given many short items
// takes fewer stages.  A (b, tile) whose stages all fall inside one workgroup
// is finished here (BF16 output + natural-log LSE); otherwise each workgroup
// writes an unreduced partial (normalised output + base-2 LSE) to one of its
// two workspace slots and the segment merge finishes the row.  The grid
// depends only on the device, the unit count only on device metadata, so the
// launch is capture-stable.
//
// Inside a workgroup: 4 waves x 32 head-rows, one wave per SIMD.  Each wave
// keeps its 32 query rows (32 x 576 BF16) in registers as the B operand of
// S^T = K Q^T (v_mfma_f32_32x32x16_bf16, A = K tile read from LDS), so a
// lane's scores all belong to one head-row and the online softmax needs one
// cross-half swap.  The probabilities P^T (rounded to BF16) stay in
// registers as the B operand of O^T = V^T P^T; the 512 x 32 output
// accumulator lives in 16 MFMA accumulators (256 AGPRs).
//
// LDS holds each 32-token stage once, as 36 blocks [32 token slots][16 BF16
// elements].  Stages arrive by direct global->LDS loads
// (global_load_lds_dwordx4): each pair of lanes owns one token row of the
// stage, so no staging registers or LDS stores are needed, and a token
// outside the sequence reads a zero row kept in the work buffer.  The PV
// operand V^T (8 tokens of one value dim per lane) is read from the same tile
// with the gfx950 transposing load ds_read_b64_tr_b16.
#include "attention_common.h"
#include "launch.h"

namespace dcpmla {

namespace {

using namespace attn;

constexpr float kRescaleSlack = 8.0f;   // keep a stale running max while 2^(s - m) <= 2^8

// LDS tile of one stage: 36 blocks of [32 token slots][16 BF16 elements],
// 36 KiB; no padding (every access pattern below covers whole 128-byte bank
// windows).
struct Tile {
  static constexpr int kRow = 32;
  static constexpr int kBlock = kStageTokens * kRow;
  static constexpr int kBytes = kKBlocks * kBlock;
  static constexpr int kLoads = kBytes / 1024;   // 1 KiB direct loads per stage
};
typedef Staging<4> Stage;   // float partials are the widest rows stored

// acc + both BF16 values of a packed pair (a dot product with (1, 1): the
// products are exact)
__device__ inline float sum_bf16_pair(uint32_t pair, float acc) {
  bf16x2 one;
  one[0] = (__bf16)1.0f;
  one[1] = (__bf16)1.0f;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// QK: v_mfma_f32_32x32x16_bf16 step j reads half h of block j, so the k-slot
// 8h + e is dim 16j + 8h + e on both operands (Q stationary, K from the tile).
__device__ inline int qdim_bf16(int j, int h) { return 16 * j + 8 * h; }

// PV operand A = V^T: lane (dim 32*dblk + l32, half h) needs tokens
// 16*kb + tau(h, e), e = 0..7, of that dim (slots 16*kb + 8h + e).  Transposing
// reads: within a 16-lane group the lane that loads address j supplies one
// row; tr_b16: result lane 4a+b, element k = element b of the row loaded by
// lane a+4k.
struct VRaw2 { short4v a, b; };

__device__ inline VRaw2 lds_v2(const uint8_t *sb, int dblk, int kb, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int h = g >> 1;
  const int kblk = 2 * dblk + (g & 1);
  const int k = j >> 2, a = j & 3;
  const uint8_t *base = sb + kblk * Tile::kBlock + 8 * a;
  const int slot0 = 16 * kb + 8 * h + k;         // tokens tau(h, k), k < 4
  const int slot1 = slot0 + 4;                   // tokens tau(h, 4 + k)
  VRaw2 r;
  r.a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v *)(lds_char *)(size_t)(base + slot0 * Tile::kRow));
  r.b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v *)(lds_char *)(size_t)(base + slot1 * Tile::kRow));
  return r;
}

__device__ inline bf16x8 widen_v(VRaw2 r) {
  // whole-vector reinterpretation (element-wise short -> __bf16 casts into a
  // vector are miscompiled to zeros by this toolchain)
  const uint2 lo = __builtin_bit_cast(uint2, r.a);
  const uint2 hi = __builtin_bit_cast(uint2, r.b);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// ---------------------------------------------------------------- staging
//
// Direct load i (1 KiB) of a stage fills tile bytes [1024 i, 1024 i + 1024);
// lane l writes 16 bytes at 1024 i + 16 l, i.e. slot l / 2, half l % 2 of
// block i: each pair of lanes reads one token row for the whole stage.
__device__ inline int stage_slot(int lane) { return lane >> 1; }
__device__ inline int stage_byte(int i, int lane) { return 32 * i + 16 * (lane & 1); }

// Address of this lane's token row for stage s (its page id prefetched one
// stage earlier), plus the lane's fixed byte offset inside the row.  A token
// past the longest row, or on a page outside the pool, reads the zero row, so
// the tile never holds stale bytes.
__device__ inline const uint8_t *stage_row(const AttnArgs &a, int32_t page, int s, int lmax, int lane,
                                           int32_t *bad) {
  const int t = s * kStageTokens + tok_slot(stage_slot(lane));
  const bool in_seq = t < lmax;
  const bool ok = page >= 0 && (int64_t)page < a.num_pages;
  *bad |= (in_seq && !ok) ? 1 : 0;
  const uint8_t *row = a.zero_row;
  if (in_seq && ok) {
    const int64_t r = ((int64_t)page << a.page_shift) + (t & ((1 << a.page_shift) - 1));
    row = a.pool + r * kDqk * 2;
  }
  return row + stage_byte(0, lane);
}

__device__ inline int32_t fetch_page(const AttnArgs &a, const int32_t *pt, int s, int lmax, int lane) {
  const int t = s * kStageTokens + tok_slot(stage_slot(lane));
  return pt[t < lmax ? (t >> a.page_shift) : 0];
}

// This wave's share of a stage: loads i = wave + 4 j.  Load i reads row bytes
// 32 i + (lane part, already in row) and fills tile bytes [1024 i, +1024).
__device__ inline void issue_stage(uint32_t tile_lds, const uint8_t *row, int wave_s) {
  constexpr int kFull = Tile::kLoads / kWaves;
  constexpr int kRest = Tile::kLoads % kWaves;
  const uint8_t *src = row + 32 * wave_s;
  const uint32_t dst = tile_lds + 1024 * wave_s;
#pragma unroll
  for (int j = 0; j < kFull; ++j) dma16(src + 128 * j, dst + 4096 * j);
  if constexpr (kRest != 0) {
    if (wave_s < kRest) dma16(src + 128 * kFull, dst + 4096 * kFull);
  }
}

// LDS: two stage tiles, the four waves' output staging areas, then
// (PartLds) the work partition and the row lengths, so locating a piece
// costs no global round trips.
template <bool PartLds>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attention_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int kslot = tok_slot(l32);   // LDS slot of the stage token in this lane's score row
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *a.ws_scale = a.out_scale;
    // fields read through kernarg_args() must be the by-value argument's
    const KernargArgs ka = kernarg_args();
    if (ka->M != a.M || ka->H != a.H || ka->err != a.err || ka->out_scale != a.out_scale)
      atomicOr(a.err, DCPMLA_ERR_KERNARG);
  }
  const int64_t U = a.work[0];
  if (U == 0) return;
  const Split sp = work_split(gridDim.x, U, a.n_mt, a.B, DCPMLA_KV_BF16);
  const int64_t G = sp.T * sp.tm;
  if ((int64_t)blockIdx.x >= G) return;
  const int64_t w = xcd_group(blockIdx.x, G);
  const int64_t team = w / sp.tm;
  const int tpos = (int)(w - team * sp.tm);   // this group's head-row tile in each team item
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_char *)lds);
  int32_t *part = (int32_t *)(lds + 2 * Tile::kBytes + Stage::kBytes);
  const int nwork = 4 * a.B + 2;
  if constexpr (PartLds) {
    for (int i = tid; i < nwork; i += kThreads) part[i] = a.work[i];
    for (int i = tid; i < a.B * a.qlen; i += kThreads) part[nwork + i] = a.row_len[i];
    __syncthreads();
  }
  Walk<PartLds> wk;
  wk.work = a.work;
  wk.part = part;
  wk.row_len = a.row_len;
  wk.B = a.B;
  wk.n_mt = sp.n_items;
  wk.tm = sp.tm;
  wk.nwork = nwork;
  wk.U = sp.cols;
  wk.pc = sp.pc;
  wk.C = sp.C;
  wk.hi = sp.cols;
  const int64_t lo = wk.units_before(group_cost_lo(team, sp.C, sp.T));
  const int64_t hi = wk.units_before(group_cost_lo(team + 1, sp.C, sp.T));
  if (lo >= hi) return;   // a cost range of piece overheads only
  wk.hi = hi;
  int32_t bad = 0;

  auto pt_of = [&](const Cursor &c) { return a.page_table + (int64_t)c.lrow * a.max_local_pages; };
  auto page_of = [&](const Cursor &c) { return fetch_page(a, pt_of(c), c.s, c.lmax, lane); };
  auto load_stage = [&](const Cursor &c, int32_t page, int buf) {
    issue_stage(lds_base + buf * Tile::kBytes, stage_row(a, page, c.s, c.lmax, lane, &bad), wave);
  };
  uint4 q[kKBlocks];   // this lane's query operand (BF16 step j)
  // this lane's head-row of the piece at c, and the query row it loads
  auto load_q = [&](const Cursor &c) {
    // lane-derived addresses and kernel arguments are re-derived per piece:
    // kept live across the piece loop they end up in scratch, and the
    // reload's wait at the top of a piece would also wait for every load and
    // store still in flight
    const int ln = fresh_lane_id();
    const KernargArgs ka = kernarg_args();
    const int M = ka->M;
    const int m = (c.mt * sp.tm + tpos) * kTileRows + wave * kWaveRows + (ln & 31);
    const bool mvalid = m < M;
    // rows past M read row M-1 (a valid address) and are zeroed
    const int64_t qr = (int64_t)c.b * M + (mvalid ? m : M - 1);
    const uint32_t keep = mvalid ? 0xFFFFFFFFu : 0u;
    const uint16_t *qrow = ka->q + qr * kDqk;
#pragma unroll
    for (int j = 0; j < kKBlocks; ++j) {
      uint4 v = *(const uint4 *)(qrow + qdim_bf16(j, ln >> 5));
      v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
      q[j] = v;
    }
  };

  Cursor P = wk.locate(lo);
  Cursor nx = P;       // cursor of the unit whose tile is in flight
  int32_t page = 0;    // page id of the unit after nx
  load_stage(P, page_of(P), 0);
  if (lo + 1 < hi) {
    nx = wk.advance(P, lo + 1);
    page = page_of(nx);
  }

  int cur = 0;
  int64_t u = lo;
  bool first_piece = true;

  while (true) {
    load_q(P);
    if (first_piece) {
      // the first tile and the first query rows are in flight together: one
      // wait covers both, then the barrier hands the tile to every wave
      wait_direct_loads();
      __syncthreads();
      first_piece = false;
    }
    // per-piece softmax state; O^T accumulates in AGPRs
    floatx16 oacc[kDv / 32];
#pragma unroll
    for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
    float mrun = kNegInf;
    float lsum = 0.f;    // sum of the BF16 probabilities fed to the PV MFMAs: normalises O
    float lsum_f = 0.f;  // fp32 sum of the same probabilities before rounding: gives the LSE
    const int b = P.b;
    const int mt = P.mt * sp.tm + tpos;   // head-row tile
    const bool complete = P.st_begin == 0 && P.st_end == P.stages;
    // this lane's head-row and its verify-row window
    const int m = mt * kTileRows + wave * kWaveRows + (fresh_lane_id() & 31);
    const bool mvalid = m < a.M;
    const int vrow = mvalid ? m / kernarg_args()->H : 0;
    // rows past M (zero queries) see every token: their results are never
    // stored, and they keep the wave on the unmasked path
    const int rlen = mvalid ? wk.row_len_at(b * a.qlen + vrow) : 0x3FFFFFFF;
    const int nst = P.st_end - P.st_begin;
    Cursor following = P;   // first unit after this piece, when there is one

    for (int k = 0; k < nst; ++k) {
      const int s = P.st_begin + k;
      const int64_t uu = u + k;
      if (uu + 1 < hi) {
        load_stage(nx, page, cur ^ 1);
        if (k == nst - 1) following = nx;
        if (uu + 2 < hi) {
          nx = wk.advance(nx, uu + 2);
          page = page_of(nx);
        }
      }
      const uint8_t *sb = lds + cur * Tile::kBytes;

      // S^T[token, row] = K Q^T over 576 dims
      floatx16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      {
        const uint8_t *kb0 = sb + kslot * Tile::kRow + 16 * h;
        uint4 kr[2];
        kr[0] = *(const uint4 *)(kb0);
        kr[1] = *(const uint4 *)(kb0 + Tile::kBlock);
#pragma unroll
        for (int j = 0; j < kKBlocks; ++j) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, kr[j & 1]);
          if (j + 2 < kKBlocks) kr[j & 1] = *(const uint4 *)(kb0 + (j + 2) * Tile::kBlock);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, __builtin_bit_cast(bf16x8, q[j]), sacc, 0, 0, 0);
        }
      }

      // online softmax in base 2 on this lane's 16 tokens of head-row m.  The
      // raw scores are kept: the max commutes with the positive scale, which
      // is applied inside the exponent.  Register r holds token
      // t0 + 4h + row_of(r) with row_of(r) = 8(r/4) + r%4 <= 27, so a stage
      // lies wholly inside every row window of the wave when
      // rlen - t0 - 4h > 27 on all lanes; only the last stages of a window
      // need the per-token mask.
      const float sc2 = a.score_scale2;
      const int t0 = s * kStageTokens;
      const int lim = rlen - t0 - 4 * h;
      float sv[16];
      if (__all(lim > 27)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = sacc[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = (8 * (r >> 2) + (r & 3)) < lim ? sacc[r] : kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[r]);
      mx = fmaxf(mx, other_half(mx, h)) * sc2;
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
      // p = 2^(score * scale - mrun); masked scores give 2^-inf = 0, and a row
      // with nothing visible yet subtracts 0 instead of -inf
      const float msub = mrun > kNegInf ? mrun : 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], sc2, -msub));
        pb[r >> 3][r & 7] = (__bf16)p;
        lsum_f += p;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 w4 = __builtin_bit_cast(uint4, pb[j]);
        lsum = sum_bf16_pair(w4.x, lsum);
        lsum = sum_bf16_pair(w4.y, lsum);
        lsum = sum_bf16_pair(w4.z, lsum);
        lsum = sum_bf16_pair(w4.w, lsum);
      }

      // O^T[d, row] += V^T[d, token] P^T[token, row]; operands prefetched two ahead
      {
        VRaw2 vr[2];
        vr[0] = lds_v2(sb, 0, 0, lane);
        vr[1] = lds_v2(sb, 0, 1, lane);
#pragma unroll
        for (int i = 0; i < kDv / 16; ++i) {
          const int d = i >> 1, kb = i & 1;
          const bf16x8 vop = widen_v(vr[i & 1]);
          if (i + 2 < kDv / 16) vr[i & 1] = lds_v2(sb, (i + 2) >> 1, (i + 2) & 1, lane);
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kb], oacc[d], 0, 0, 0);
        }
      }

      // the next unit's direct loads (this wave's share) have landed; the
      // barrier makes every wave's share visible and frees the current tile
      wait_direct_loads();
      __syncthreads();
      cur ^= 1;
    }
    u += nst;
    const bool more = u < hi;
    // finish the piece
    const float ltot = lsum + other_half(lsum, h);
    const float ltot_f = lsum_f + other_half(lsum_f, h);
    const bool has = ltot > 0.f;
    const float inv = has ? a.out_scale / ltot : 0.f;
    const float lse2 = has ? mrun + __builtin_amdgcn_logf(ltot_f) : kNegInf;
    // rows of this wave that exist (m < M)
    const int nrows = min(kWaveRows, a.M - (mt * kTileRows + wave * kWaveRows));
    uint8_t *stg = lds + 2 * Tile::kBytes + wave * Stage::kWaveBytes;
    // output pointers are read where they are used (see kernarg_args)
    const KernargArgs ka = kernarg_args();
    if (complete) {
      __bf16 *orow0 = (__bf16 *)ka->out + ((int64_t)b * a.M + mt * kTileRows + wave * kWaveRows) * kDv;
      store_rows<4>(oacc, inv, stg, orow0, nrows);
      if (mvalid && h == 0)
        ka->lse[(int64_t)b * a.M + mt * kTileRows + wave * kWaveRows + (fresh_lane_id() & 31)] =
            has ? lse2 * kLn2 : kNegInf;
    } else {
      // rows past M are never merged: no partial for them
      const int64_t prow0 = (w * kSlots + piece_slot(P.st_begin)) * kTileRows + wave * kWaveRows;
      store_rows<4>(oacc, inv, stg, (float *)ka->ws_o + prow0 * kDv, nrows);
      if (mvalid && h == 0) ka->ws_lse2[prow0 + (fresh_lane_id() & 31)] = lse2;
    }
    if (!more) break;
    P = following;
  }
  if (bad) atomicOr(a.err, DCPMLA_ERR_PAGE_RANGE);
}

constexpr size_t kLdsLimit = 160 * 1024;   // gfx950 LDS per workgroup

// The dynamic-LDS cap is raised once per device (the attribute is per device).
template <bool PartLds>
hipError_t launch_variant(const AttnArgs &a, int groups, size_t shmem, hipStream_t stream) {
  static DeviceOnce once;
  const size_t cap = PartLds ? kLdsLimit : 2 * Tile::kBytes + Stage::kBytes;
  const hipError_t e = once.run([&] {
    return hipFuncSetAttribute((const void *)attention_kernel<PartLds>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)cap);
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attention_kernel<PartLds>), dim3(groups), dim3(kThreads), shmem, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const AttnArgs &args, int groups, hipStream_t stream) {
  AttnArgs a = args;
  const size_t tiles = 2 * Tile::kBytes + Stage::kBytes;
  const size_t part = (size_t)(4 * (int64_t)a.B + 2 + (int64_t)a.B * a.qlen) * 4;
  if (tiles + part <= kLdsLimit) {
    a.part_ints = (int)(part / 4);
    return launch_variant<true>(a, groups, tiles + part, stream);
  }
  a.part_ints = 0;
  return launch_variant<false>(a, groups, tiles, stream);
}

hipError_t launch_partial_attention(const dcpmla_geom &g, int groups, const void *q,
                                    const void *q_split, const float *q_inv_scale,
                                    const void *kv_pool, float kv_scale, float softmax_scale,
                                    const dcpmla_meta &m, void *workspace, void *out_rank,
                                    float *lse_rank, hipStream_t stream) {
  AttnArgs a;
  a.q = (const uint16_t *)q;
  a.pool = (const uint8_t *)kv_pool;
  a.zero_row = (const uint8_t *)(m.work + work_zero_off(g.batch));
  a.row_len = m.row_local_len;
  a.page_table = m.page_table;
  a.work = m.work;
  a.qsplit = nullptr;
  a.qscale = nullptr;
  a.ws_o = workspace;
  a.ws_lse2 = (float *)workspace + ws_o_floats(groups);
  a.ws_scale = (float *)workspace + ws_scale_off(groups);
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
  a.part_ints = 0;
  a.kv_dtype = g.kv_dtype;
  a.score_scale2 = softmax_scale * kv_scale * 1.44269504088896340736f;
  a.out_scale = kv_scale;
  if (g.kv_dtype != DCPMLA_KV_FP8_E4M3) return launch_attention_bf16(a, groups, stream);
  const int64_t rows = (int64_t)g.batch * a.M;
  if (q_split) {
    // the caller's split query
    a.qsplit = (const uint8_t *)q_split;
    a.qscale = q_inv_scale;
  } else {
    // the query as two E4M3 terms for the FP8 products, then the attention
    a.qsplit = (const uint8_t *)workspace + ws_qsplit_off(groups);
    a.qscale = (const float *)((const uint8_t *)workspace + ws_qscale_off(groups, rows));
    const hipError_t e = launch_split_q(rows, q, (uint8_t *)workspace + ws_qsplit_off(groups),
                                        (float *)((uint8_t *)workspace + ws_qscale_off(groups, rows)), stream);
    if (e != hipSuccess) return e;
  }
  return launch_attention_fp8(a, groups, g.q_format == DCPMLA_Q_FP8, g.p_format == DCPMLA_P_FP8, stream);
}

}  // namespace dcpmla
