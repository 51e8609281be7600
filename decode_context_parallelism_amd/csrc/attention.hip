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
// cross-half swap.  The probabilities P^T stay in registers as the B operand
// of O^T = V^T P^T; the 512 x 32 output accumulator lives in 16 MFMA
// accumulators (256 AGPRs).
//
// LDS holds each 32-token stage once, in the cache's own element format, as
// 36 blocks [16 dims][32 token slots][16 elements].  Stages arrive by direct
// global->LDS loads (global_load_lds_dwordx4): each lane owns one token row of
// the stage, so no staging registers or LDS stores are needed, and a token
// outside the sequence reads a zero row kept in the work buffer.  The QK
// operand is a plain row read of the tile; the PV operand V^T (8 tokens of
// one value dim per lane) is read from the same tile with the gfx950
// transposing loads ds_read_b64_tr_b8 / ds_read_b64_tr_b16, so no transposed
// copy of V is kept.  FP8 elements are widened to BF16 in registers right
// before each MFMA; E4M3 -> BF16 is exact, so the kv scale folds into the
// score scale and the output.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace dcpmla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // keep a stale running max while 2^(s - m) <= 2^8

constexpr int kKBlocks = kDqk / 16;     // 36 blocks of 16 dims

struct AttnArgs {
  const uint16_t *q;         // [B, qlen, H, 576] bf16 bits
  const uint8_t *pool;       // [num_pages * P, 576] cache elements
  const uint8_t *zero_row;   // 576 zero elements (either format)
  const int32_t *row_len;    // [B*qlen]
  const int32_t *page_table; // [B*qlen, max_local_pages]
  const int32_t *work;
  const uint8_t *qsplit;     // FP8 cache: [B*M][2][576] E4M3 codes hi, lo of the query
  const float *qscale;       // FP8 cache: [B*M] 2^-k, q = (hi + lo) * 2^-k
  void *ws_o;                // [G][2][128][512] fp16 (FP8 cache) or float (BF16 cache)
  float *ws_lse2;            // [G][2][128]
  float *ws_scale;           // scale of the fp16 partials
  uint16_t *out;             // [B, qlen, H, 512] bf16 bits
  float *lse;                // [B, qlen, H]
  int32_t *err;
  int64_t num_pages;
  int B, qlen, H, M, n_mt, page_shift, max_local_pages;
  int part_ints;             // 4B+2 partition ints + B*qlen row lengths (staged in LDS)
  float score_scale2;        // softmax_scale * kv_scale * log2(e)
  float out_scale;           // kv_scale
};

// This lane's index in the wave, read from the hardware at each call (a
// volatile asm the compiler can neither hoist nor keep live across loops:
// recomputing it is cheaper than a register held through the stage loop).
__device__ inline int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The kernel's argument block as it sits in the kernel-argument segment
// (attention_kernel takes its AttnArgs by value as its only argument, so the
// block starts at offset 0).  Reading a field through this pointer is a
// scalar load; the empty asm makes each call a fresh pointer, so the compiler
// re-reads the field where it is used instead of holding it in registers
// across the kernel.
typedef const __attribute__((address_space(4))) AttnArgs *KernargArgs;
__device__ inline KernargArgs kernarg_args() {
  KernargArgs p = (KernargArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// LDS tile of one stage with E-byte elements: 36 blocks of [32 token slots]
// [16 elements], 18 KiB (FP8) or 36 KiB (BF16); no padding (every access
// pattern below covers whole 128-byte bank windows).
template <int E>
struct Tile {
  static constexpr int kRow = 16 * E;
  static constexpr int kBlock = kStageTokens * kRow;
  static constexpr int kBytes = kKBlocks * kBlock;
  static constexpr int kLoads = kBytes / 1024;   // 1 KiB direct loads per stage
};

// Accumulator layout: register r of a 32x32 accumulator in lane half h holds
// row 8*(r/4) + 4*h + r%4 of the MFMA output tile, so in the score tile it
// holds that token of the stage.  The same map assigns PV k-slot 8*h + e
// (e < 8) of token half kb to token 16*kb + tau(h, e).

// LDS row slot of stage-token t (and, being an involution -- it swaps bits 2
// and 3 -- the token of slot t).  The PV operand of lane half h gathers the
// eight tokens tau(h, 0..7) = {4h..4h+3, 8+4h..8+4h+3} (+16 for the second
// token half); storing those eight rows in consecutive slots 8h..8h+7 makes
// each 16-lane transposing read touch every bank exactly once.
__host__ __device__ inline int tok_slot(int t) {
  return 16 * (t >> 4) + 8 * ((t >> 2) & 1) + 4 * ((t >> 3) & 1) + (t & 3);
}

// Value of lane l ^ 32 (the other half of the 32x32 accumulator column),
// from v_permlane32_swap: it exchanges the upper half of its first operand
// with the lower half of its second, so for lanes below 32 the second result
// holds the upper half's value and for the others the first result holds the
// lower half's.  The first operand goes through an empty asm so the compiler
// sees two distinct inputs and keeps both results.
__device__ inline float other_half(float x, int h) {
  uint32_t y = __builtin_bit_cast(uint32_t, x);
  asm volatile("" : "+v"(y));
  const auto r = __builtin_amdgcn_permlane32_swap(y, __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, h ? r[0] : r[1]);
}

// acc + both BF16 values of a packed pair (a dot product with (1, 1): the
// products are exact)
__device__ inline float sum_bf16_pair(uint32_t pair, float acc) {
  bf16x2 one;
  one[0] = (__bf16)1.0f;
  one[1] = (__bf16)1.0f;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

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

// ------------------------------------------------------------ QK operands
//
// Q is the stationary B operand, K (from the tile) the A operand; both map
// their k-slots to the same dims (any map works as long as they agree).
//   FP8 tile: S^T = K hi + K lo on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3,
//     fp32 accumulate).  Step t, lane half h, byte e (0..31) is dim
//     64t + 32h + e: 32 contiguous bytes of the token row, i.e. tile blocks
//     4t + 2h and 4t + 2h + 1, and the same 32 bytes of the split query's hi
//     and lo codes.  The cache elements go to the matrix unit as stored.
//   BF16 tile: v_mfma_f32_32x32x16_bf16 step j reads half h of block j, so
//     the k-slot 8h + e is dim 16j + 8h + e.
__device__ inline int qdim_bf16(int j, int h) { return 16 * j + 8 * h; }

__device__ inline int8v cat8(uint4 a, uint4 b) {
  int8v r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

// per-lane query operand registers
template <int E> struct QOperand;
template <> struct QOperand<1> { int8v v[2 * (kDqk / 64)]; };   // hi, lo of each 64-dim step
template <> struct QOperand<2> { uint4 v[kKBlocks]; };           // bf16 step j

// ------------------------------------------------------------ PV operands
//
// A = V^T: lane (dim 32*dblk + l32, half h) needs tokens 16*kb + tau(h, e),
// e = 0..7, of that dim (slots 16*kb + 8h + e).  Transposing reads: within a
// 16-lane group the lane that loads address j supplies one row;
//   tr_b8:  result lane 8a+b, byte k = byte b of the row loaded by lane a+2k;
//   tr_b16: result lane 4a+b, element k = element b of the row loaded by a+4k.
__device__ inline int2v lds_v1(const uint8_t *sb, int dblk, int kb, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int h = g >> 1;
  const int kblk = 2 * dblk + (g & 1);
  const int k = j >> 1, a = j & 1;
  const int slot = 16 * kb + 8 * h + k;
  const uint8_t *p = sb + kblk * Tile<1>::kBlock + slot * Tile<1>::kRow + 8 * a;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) int2v *)(lds_char *)(size_t)p);
}

struct VRaw2 { short4v a, b; };

__device__ inline VRaw2 lds_v2(const uint8_t *sb, int dblk, int kb, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int h = g >> 1;
  const int kblk = 2 * dblk + (g & 1);
  const int k = j >> 2, a = j & 3;
  const uint8_t *base = sb + kblk * Tile<2>::kBlock + 8 * a;
  const int slot0 = 16 * kb + 8 * h + k;         // tokens tau(h, k), k < 4
  const int slot1 = slot0 + 4;                   // tokens tau(h, 4 + k)
  VRaw2 r;
  r.a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v *)(lds_char *)(size_t)(base + slot0 * Tile<2>::kRow));
  r.b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v *)(lds_char *)(size_t)(base + slot1 * Tile<2>::kRow));
  return r;
}

__device__ inline bf16x8 widen_v(int2v r) {
  return widen_fp8(make_uint2((uint32_t)r[0], (uint32_t)r[1]));
}
__device__ inline bf16x8 widen_v(VRaw2 r) {
  // whole-vector reinterpretation (element-wise short -> __bf16 casts into a
  // vector are miscompiled to zeros by this toolchain)
  const uint2 lo = __builtin_bit_cast(uint2, r.a);
  const uint2 hi = __builtin_bit_cast(uint2, r.b);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

template <int E>
struct VOp { typedef typename std::conditional<E == 1, int2v, VRaw2>::type Raw; };

template <int E>
__device__ inline typename VOp<E>::Raw lds_v(const uint8_t *sb, int dblk, int kb, int lane) {
  if constexpr (E == 1) return lds_v1(sb, dblk, kb, lane);
  else return lds_v2(sb, dblk, kb, lane);
}

// ---------------------------------------------------------------- staging
//
// Direct load i (1 KiB) of a stage fills tile bytes [1024 i, 1024 i + 1024);
// lane l writes 16 bytes at 1024 i + 16 l.  With the tile layout above that
// is slot l % 32 of blocks 2i, 2i+1 (FP8) or slot l / 2, half l % 2 of block
// i (BF16): each lane reads one token row for the whole stage.
template <int E>
__device__ inline int stage_slot(int lane) { return E == 1 ? (lane & 31) : (lane >> 1); }

template <int E>
__device__ inline int stage_byte(int i, int lane) {   // byte offset inside the token row
  return E == 1 ? 16 * (2 * i + (lane >> 5)) : 32 * i + 16 * (lane & 1);
}

// Address of this lane's token row for stage s (its page id prefetched one
// stage earlier), plus the lane's fixed byte offset inside the row.  A token
// past the longest row, or on a page outside the pool, reads the zero row, so
// the tile never holds stale bytes (an FP8 NaN pattern times a zero
// probability would poison the output).
template <int E>
__device__ inline const uint8_t *stage_row(const AttnArgs &a, int32_t page, int s, int lmax,
                                           int lane, int32_t *bad) {
  const int t = s * kStageTokens + tok_slot(stage_slot<E>(lane));
  const bool in_seq = t < lmax;
  const bool ok = page >= 0 && (int64_t)page < a.num_pages;
  *bad |= (in_seq && !ok) ? 1 : 0;
  const uint8_t *row = a.zero_row;
  if (in_seq && ok) {
    const int64_t r = ((int64_t)page << a.page_shift) + (t & ((1 << a.page_shift) - 1));
    row = a.pool + r * kDqk * E;
  }
  return row + stage_byte<E>(0, lane);
}

template <int E>
__device__ inline int32_t fetch_page(const AttnArgs &a, const int32_t *pt, int s, int lmax, int lane) {
  const int t = s * kStageTokens + tok_slot(stage_slot<E>(lane));
  return pt[t < lmax ? (t >> a.page_shift) : 0];
}

// One direct load: 64 lanes x 16 bytes from src (per lane) to LDS bytes
// [lds_addr + 16 lane].  M0 carries the wave-uniform LDS address (one wait
// state between its write and the load); the block restores the caller's M0,
// which the compiler treats as a reserved register.  Issued from asm so the
// compiler does not pair every later LDS read with a wait on these loads (it
// cannot tell the stage tiles apart); completion is awaited explicitly before
// the barrier that hands a tile to the other waves.
__device__ inline void dma16(const uint8_t *src, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// This wave's share of a stage: loads i = wave + 4 j.  Load i reads row bytes
// 32 i + (lane part, already in row) and fills tile bytes [1024 i, +1024).
// The loads of one call share one M0 save/restore (the instruction offset
// stays 0, as it would move the LDS side too).
template <int E>
__device__ inline void issue_stage(uint32_t tile_lds, const uint8_t *row, int wave_s) {
  constexpr int kFull = Tile<E>::kLoads / kWaves;
  constexpr int kRest = Tile<E>::kLoads % kWaves;
  const uint8_t *src = row + 32 * wave_s;
  const uint32_t dst = tile_lds + 1024 * wave_s;
  if constexpr (kFull == 4) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %6\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %7\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, off\n\t"
        "s_mov_b32 m0, %8\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "v"(src + 128), "v"(src + 256), "v"(src + 384),
          "s"(dst), "s"(dst + 4096), "s"(dst + 8192), "s"(dst + 12288)
        : "memory");
  } else {
#pragma unroll
    for (int j = 0; j < kFull; ++j) dma16(src + 128 * j, dst + 4096 * j);
  }
  if constexpr (kRest != 0) {
    if (wave_s < kRest) dma16(src + 128 * kFull, dst + 4096 * kFull);
  }
}

__device__ inline void wait_direct_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Word 3 of a raw (unswizzled, stride 0) buffer resource: 32-bit data
// format, all other fields zero; num_records then counts bytes.
constexpr int kRawBufferFlags = 0x00020000;

// Output staging.  The accumulator leaves the MFMA with 4 consecutive dims of
// one head-row per lane, so storing it directly would touch 32 rows per
// store.  Instead each wave moves its 32 x 512 block in passes of 128 dims
// through its own LDS area: written in the accumulator layout, read back as
// 16-byte pieces of rows, and stored as whole 256- or 512-byte row segments.
// Rows are padded by 16 bytes so the accumulator-layout writes spread over
// all banks.  Waves never share an area, so no barrier is needed.
template <int E>
struct Staging {
  static constexpr int kPassDims = 128;
  static constexpr int kRowBytes = kPassDims * (E == 1 ? 2 : 4) + 16;   // widest element stored
  static constexpr int kWaveBytes = kWaveRows * kRowBytes;
  static constexpr int kBytes = kWaves * kWaveBytes;
};

// rows[r * kDv + c] = T(acc(row r, dim c) * sc) for rows r < nrows; T is
// __bf16, _Float16 or float.  The row stores are raw buffer stores whose
// resource covers only the nrows valid rows, so rows past the end are
// dropped by the range check instead of being branched around: a branch per
// store makes the compiler keep values across it in scratch, and each
// reload's wait would then also wait for every store issued before it.
template <int E, typename T>
__device__ inline void store_rows(const floatx16 (&acc)[kDv / 32], float sc, uint8_t *stg, T *rows,
                                  int nrows) {
  constexpr int kRow = Staging<E>::kRowBytes;
  constexpr int kSegBytes = Staging<E>::kPassDims * (int)sizeof(T);
  constexpr int kLanesPerRow = kSegBytes / 16;
  constexpr int kRowsPerRead = 64 / kLanesPerRow;
  constexpr int kRowBytes = kDv * (int)sizeof(T);
  // addresses derived from the lane are recomputed per call, not hoisted
  // out of the piece loop (where they would stay live through the stages)
  const int lane = fresh_lane_id();
  const int l32 = lane & 31, h = lane >> 5;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(rows, (short)0, nrows > 0 ? nrows * kRowBytes : 0, kRawBufferFlags);
  const int rlane = lane / kLanesPerRow, c = lane % kLanesPerRow;
#pragma unroll
  for (int pass = 0; pass < kDv / Staging<E>::kPassDims; ++pass) {
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      const int d = 4 * pass + dd;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint8_t *dst = stg + l32 * kRow + (32 * dd + 8 * g4 + 4 * h) * (int)sizeof(T);
        const float v0 = acc[d][4 * g4 + 0] * sc, v1 = acc[d][4 * g4 + 1] * sc;
        const float v2 = acc[d][4 * g4 + 2] * sc, v3 = acc[d][4 * g4 + 3] * sc;
        if constexpr (sizeof(T) == 4) {
          *(float4 *)dst = make_float4(v0, v1, v2, v3);
        } else {
          const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (T)v0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (T)v1) << 16);
          const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (T)v2) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (T)v3) << 16);
          *(uint2 *)dst = make_uint2(w0, w1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < kWaveRows / kRowsPerRead; ++i) {
      const int r = i * kRowsPerRead + rlane;
      const int4v v = *(const int4v *)(stg + r * kRow + 16 * c);
      __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, r * kRowBytes + pass * kSegBytes + 16 * c, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// LDS: two stage tiles, the four waves' output staging areas, then
// (PartLds) the work partition and the row lengths, so locating a piece
// costs no global round trips.
template <int E, bool PartLds, bool QF8>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attention_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int kslot = tok_slot(l32);   // LDS slot of the stage token in this lane's score row
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.ws_scale = a.out_scale;
  const int64_t U = a.work[0];
  if (U == 0) return;
  const int64_t G = effective_groups(gridDim.x, U);
  if ((int64_t)blockIdx.x >= G) return;
  const int64_t w = xcd_group(blockIdx.x, G);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_char *)lds);
  int32_t *part = (int32_t *)(lds + 2 * Tile<E>::kBytes + Staging<E>::kBytes);
  const int nwork = 4 * a.B + 2;
  if constexpr (PartLds) {
    for (int i = tid; i < nwork; i += kThreads) part[i] = a.work[i];
    for (int i = tid; i < a.B * a.qlen; i += kThreads) part[nwork + i] = a.row_len[i];
    __syncthreads();
  }
  // partition values are the same for the whole workgroup: keep them in
  // scalar registers
  auto work_at = [&](int i) -> int32_t {
    if constexpr (PartLds) return __builtin_amdgcn_readfirstlane(part[i]);
    else return __builtin_amdgcn_readfirstlane(a.work[i]);
  };
  auto row_len_at = [&](int i) -> int32_t {
    if constexpr (PartLds) return part[nwork + i];
    else return a.row_len[i];
  };
  // units whose cost position is below x (the unit index at cost x)
  const int64_t C = total_cost(U, a.n_mt, a.B);
  auto units_before = [&](int64_t x) -> int64_t {
    if (x >= C) return U;
    int blo = 0, bhi = a.B;   // seq_cost(blo) <= x < seq_cost(bhi)
    while (bhi - blo > 1) {
      const int mid = (blo + bhi) >> 1;
      if (seq_cost(work_at(work_unit_base_off() + mid), a.n_mt, mid) <= x) blo = mid; else bhi = mid;
    }
    const int64_t base = work_at(work_unit_base_off() + blo);
    const int64_t st = work_at(work_stages_off(a.B) + blo);
    const int64_t rem = x - seq_cost(base, a.n_mt, blo);
    const int64_t mt = rem / (st + kPieceCost);
    const int64_t off = rem - mt * (st + kPieceCost) - kPieceCost;
    return base + mt * st + (off > 0 ? off : 0);
  };
  const int64_t lo = units_before(group_cost_lo(w, C, G));
  const int64_t hi = units_before(group_cost_lo(w + 1, C, G));
  if (lo >= hi) return;   // a cost range of piece overheads only
  int32_t bad = 0;

  // The group's units [lo, hi) are walked as one stream of (piece, stage)
  // cursors.  A piece is one (sequence, tile) and the run of its stages this
  // group owns; the tile of the next unit -- in this piece or the next --
  // is loaded while the current one is computed, so a new piece waits only
  // for its query rows.
  struct Cursor {
    int b, mt, s;          // sequence, head-row tile, stage
    int st_begin, st_end;  // this group's stages of the piece
    int stages;            // stages of sequence b
    int lmax, lrow;        // b's longest rank-local row length and the row that has it
  };
  // per-sequence values, read once when a cursor reaches a sequence (not per stage)
  auto enter_seq = [&](Cursor &c) {
    c.stages = work_at(work_stages_off(a.B) + c.b);
    c.lmax = work_at(work_lmax_off(a.B) + c.b);
    c.lrow = work_at(work_lrow_off(a.B) + c.b);
  };
  auto locate = [&](int64_t u) {
    int blo = 0, bhi = a.B;   // unit_base[blo] <= u < unit_base[bhi]
    while (bhi - blo > 1) {
      const int mid = (blo + bhi) >> 1;
      if ((int64_t)work_at(work_unit_base_off() + mid) <= u) blo = mid; else bhi = mid;
    }
    Cursor c;
    c.b = blo;
    enter_seq(c);
    const int64_t rem = u - work_at(work_unit_base_off() + blo);
    c.mt = (int)(rem / c.stages);
    c.s = (int)(rem - (int64_t)c.mt * c.stages);
    c.st_begin = c.s;
    c.st_end = (int)min((int64_t)c.stages, c.s + (hi - u));
    return c;
  };
  // cursor of unit u + 1 from that of unit u (u + 1 < hi)
  auto advance = [&](Cursor c, int64_t u_next) {
    if (++c.s < c.st_end) return c;
    if (++c.mt >= a.n_mt) {
      c.mt = 0;
      do { ++c.b; } while (work_at(work_stages_off(a.B) + c.b) == 0);
      enter_seq(c);
    }
    c.s = 0;
    c.st_begin = 0;
    c.st_end = (int)min((int64_t)c.stages, hi - u_next);
    return c;
  };
  auto lmax_of = [&](const Cursor &c) { return c.lmax; };
  auto pt_of = [&](const Cursor &c) { return a.page_table + (int64_t)c.lrow * a.max_local_pages; };
  auto page_of = [&](const Cursor &c) { return fetch_page<E>(a, pt_of(c), c.s, lmax_of(c), lane); };
  auto load_stage = [&](const Cursor &c, int32_t page, int buf) {
    issue_stage<E>(lds_base + buf * Tile<E>::kBytes, stage_row<E>(a, page, c.s, lmax_of(c), lane, &bad), wave);
  };
  // the query operand, 576 bytes per lane in either format (FP8 cache: step
  // t's hi codes in q.v[2t], lo codes in q.v[2t+1])
  QOperand<E> q;
  float sc2 = a.score_scale2;   // this lane's score scale (times 2^-k with a split query)
  // this lane's head-row of the piece at c, and the query row it loads
  auto load_q = [&](const Cursor &c) {
    // lane-derived addresses are recomputed per piece: kept live across the
    // piece loop they end up in scratch, and the reload's wait at the top of
    // a piece would also wait for every load and store still in flight
    const int ln = fresh_lane_id();
    // the arguments it needs are read again from the kernel-argument segment
    // (scalar loads), not kept in registers from the kernel's start
    const KernargArgs ka = kernarg_args();
    const int M = ka->M;
    const int m = c.mt * kTileRows + wave * kWaveRows + (ln & 31);
    const bool mvalid = m < M;
    // rows past M read row M-1 (a valid address) and are zeroed
    const int64_t qr = (int64_t)c.b * M + (mvalid ? m : M - 1);
    const uint32_t keep = mvalid ? 0xFFFFFFFFu : 0u;
    if constexpr (E == 1) {
      // tiled split: chunk 4t + 2 term + half holds this lane's 16 bytes at
      // 16 (32 h + row % 32), so each load below reads one contiguous KiB
      // across the wave (two runs when a wave's rows straddle a 32-row block)
      const uint8_t *qrow = ka->qsplit + qsplit_off(qr, 0, ln >> 5);
#pragma unroll
      for (int t = 0; t < kDqk / 64; ++t) {
        q.v[2 * t] = cat8(*(const uint4 *)(qrow + (4 * t) * kQSplitChunk),
                          *(const uint4 *)(qrow + (4 * t + 1) * kQSplitChunk));
        q.v[2 * t + 1] = cat8(*(const uint4 *)(qrow + (4 * t + 2) * kQSplitChunk),
                              *(const uint4 *)(qrow + (4 * t + 3) * kQSplitChunk));
      }
#pragma unroll
      for (int j = 0; j < 2 * (kDqk / 64); ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) q.v[j][e] &= (int)keep;
      sc2 = ka->score_scale2 * ka->qscale[qr];
    } else {
      const uint16_t *qrow = ka->q + qr * kDqk;
#pragma unroll
      for (int j = 0; j < kKBlocks; ++j) {
        uint4 v = *(const uint4 *)(qrow + qdim_bf16(j, ln >> 5));
        v.x &= keep; v.y &= keep; v.z &= keep; v.w &= keep;
        q.v[j] = v;
      }
    }
  };

  Cursor P = locate(lo);
  Cursor nx = P;       // cursor of the unit whose tile is in flight
  int32_t page = 0;    // page id of the unit after nx
  load_stage(P, page_of(P), 0);
  if (lo + 1 < hi) {
    nx = advance(P, lo + 1);
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
    const int mt = P.mt;
    const bool complete = P.st_begin == 0 && P.st_end == P.stages;
    // this lane's head-row and its verify-row window (lane and head count
    // re-read here, for the reason given at kernarg_args)
    const int m = mt * kTileRows + wave * kWaveRows + (fresh_lane_id() & 31);
    const bool mvalid = m < a.M;
    const int vrow = mvalid ? m / kernarg_args()->H : 0;
    // rows past M (zero queries) see every token: their results are never
    // stored, and they keep the wave on the unmasked path
    const int rlen = mvalid ? row_len_at(b * a.qlen + vrow) : 0x3FFFFFFF;
    const int nst = P.st_end - P.st_begin;
    Cursor following = P;   // first unit after this piece, when there is one

    for (int k = 0; k < nst; ++k) {
      const int s = P.st_begin + k;
      const int64_t uu = u + k;
      if (uu + 1 < hi) {
        load_stage(nx, page, cur ^ 1);
        if (k == nst - 1) following = nx;
        if (uu + 2 < hi) {
          nx = advance(nx, uu + 2);
          page = page_of(nx);
        }
      }
      const uint8_t *sb = lds + cur * Tile<E>::kBytes;

      // S^T[token, row] = K Q^T over 576 dims
      floatx16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      if constexpr (E == 1) {
        // Per step t two 16-byte tile reads (blocks 4t + 2h, 4t + 2h + 1: 32
        // dims of this lane's token row) feed the hi and the lo product.  Written
        // out so the reads run two steps ahead of the MFMAs in three fixed
        // register tuples and the scores stay in VGPRs; the compiler left alone
        // waits for each step's reads and moves an output block out of the
        // AGPRs to hold the scores.  The closing nops are the wait states an
        // XDL result needs before a VALU reads it.
        const uint32_t kaddr = lds_base + cur * Tile<1>::kBytes + 2 * h * Tile<1>::kBlock + kslot * Tile<1>::kRow;
        if constexpr (!QF8) {
          asm volatile(
              "s_waitcnt lgkmcnt(0)\n\t"
              "ds_read_b128 v[240:243], %[addr] offset:0\n\t"
              "ds_read_b128 v[244:247], %[addr] offset:512\n\t"
              "ds_read_b128 v[248:251], %[addr] offset:2048\n\t"
              "ds_read_b128 v[252:255], %[addr] offset:2560\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q0], 0\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q1], %[acc]\n\t"
              "ds_read_b128 v[232:235], %[addr] offset:4096\n\t"
              "ds_read_b128 v[236:239], %[addr] offset:4608\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q2], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q3], %[acc]\n\t"
              "ds_read_b128 v[240:243], %[addr] offset:6144\n\t"
              "ds_read_b128 v[244:247], %[addr] offset:6656\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q4], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q5], %[acc]\n\t"
              "ds_read_b128 v[248:251], %[addr] offset:8192\n\t"
              "ds_read_b128 v[252:255], %[addr] offset:8704\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q6], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q7], %[acc]\n\t"
              "ds_read_b128 v[232:235], %[addr] offset:10240\n\t"
              "ds_read_b128 v[236:239], %[addr] offset:10752\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q8], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q9], %[acc]\n\t"
              "ds_read_b128 v[240:243], %[addr] offset:12288\n\t"
              "ds_read_b128 v[244:247], %[addr] offset:12800\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q10], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q11], %[acc]\n\t"
              "ds_read_b128 v[248:251], %[addr] offset:14336\n\t"
              "ds_read_b128 v[252:255], %[addr] offset:14848\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q12], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q13], %[acc]\n\t"
              "ds_read_b128 v[232:235], %[addr] offset:16384\n\t"
              "ds_read_b128 v[236:239], %[addr] offset:16896\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q14], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q15], %[acc]\n\t"
              "s_waitcnt lgkmcnt(0)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q16], %[acc]\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q17], %[acc]\n\t"
              "s_nop 15\n\t"
              "s_nop 3\n\t"
              : [acc] "=&v"(sacc)
              : [addr] "v"(kaddr), [q0] "v"(q.v[0]), [q1] "v"(q.v[1]), [q2] "v"(q.v[2]), [q3] "v"(q.v[3]), [q4] "v"(q.v[4]), [q5] "v"(q.v[5]), [q6] "v"(q.v[6]), [q7] "v"(q.v[7]), [q8] "v"(q.v[8]), [q9] "v"(q.v[9]), [q10] "v"(q.v[10]), [q11] "v"(q.v[11]), [q12] "v"(q.v[12]), [q13] "v"(q.v[13]), [q14] "v"(q.v[14]), [q15] "v"(q.v[15]), [q16] "v"(q.v[16]), [q17] "v"(q.v[17])
              : "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255", "memory");
        } else {
          // the quantised query: the hi terms alone
          asm volatile(
              "s_waitcnt lgkmcnt(0)\n\t"
              "ds_read_b128 v[240:243], %[addr] offset:0\n\t"
              "ds_read_b128 v[244:247], %[addr] offset:512\n\t"
              "ds_read_b128 v[248:251], %[addr] offset:2048\n\t"
              "ds_read_b128 v[252:255], %[addr] offset:2560\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q0], 0\n\t"
              "ds_read_b128 v[232:235], %[addr] offset:4096\n\t"
              "ds_read_b128 v[236:239], %[addr] offset:4608\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q2], %[acc]\n\t"
              "ds_read_b128 v[240:243], %[addr] offset:6144\n\t"
              "ds_read_b128 v[244:247], %[addr] offset:6656\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q4], %[acc]\n\t"
              "ds_read_b128 v[248:251], %[addr] offset:8192\n\t"
              "ds_read_b128 v[252:255], %[addr] offset:8704\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q6], %[acc]\n\t"
              "ds_read_b128 v[232:235], %[addr] offset:10240\n\t"
              "ds_read_b128 v[236:239], %[addr] offset:10752\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q8], %[acc]\n\t"
              "ds_read_b128 v[240:243], %[addr] offset:12288\n\t"
              "ds_read_b128 v[244:247], %[addr] offset:12800\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q10], %[acc]\n\t"
              "ds_read_b128 v[248:251], %[addr] offset:14336\n\t"
              "ds_read_b128 v[252:255], %[addr] offset:14848\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[240:247], %[q12], %[acc]\n\t"
              "ds_read_b128 v[232:235], %[addr] offset:16384\n\t"
              "ds_read_b128 v[236:239], %[addr] offset:16896\n\t"
              "s_waitcnt lgkmcnt(2)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[248:255], %[q14], %[acc]\n\t"
              "s_waitcnt lgkmcnt(0)\n\t"
              "v_mfma_f32_32x32x64_f8f6f4 %[acc], v[232:239], %[q16], %[acc]\n\t"
              "s_nop 15\n\t"
              "s_nop 3\n\t"
              : [acc] "=&v"(sacc)
              : [addr] "v"(kaddr), [q0] "v"(q.v[0]), [q2] "v"(q.v[2]), [q4] "v"(q.v[4]), [q6] "v"(q.v[6]), [q8] "v"(q.v[8]), [q10] "v"(q.v[10]), [q12] "v"(q.v[12]), [q14] "v"(q.v[14]), [q16] "v"(q.v[16])
              : "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255", "memory");
        }
      } else {
        const uint8_t *kb0 = sb + kslot * Tile<2>::kRow + 16 * h;
        uint4 kr[2];
        kr[0] = *(const uint4 *)(kb0);
        kr[1] = *(const uint4 *)(kb0 + Tile<2>::kBlock);
#pragma unroll
        for (int j = 0; j < kKBlocks; ++j) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, kr[j & 1]);
          if (j + 2 < kKBlocks) kr[j & 1] = *(const uint4 *)(kb0 + (j + 2) * Tile<2>::kBlock);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, __builtin_bit_cast(bf16x8, q.v[j]), sacc, 0, 0, 0);
        }
      }

      // online softmax in base 2 on this lane's 16 tokens of head-row m.  The
      // raw scores are kept: the max commutes with the positive scale, which
      // is applied inside the exponent.  Register r holds token
      // t0 + 4h + row_of(r) with row_of(r) = 8(r/4) + r%4 <= 27, so a stage
      // lies wholly inside every row window of the wave when
      // rlen - t0 - 4h > 27 on all lanes; only the last stages of a window
      // need the per-token mask.
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
        typename VOp<E>::Raw vr[2];
        vr[0] = lds_v<E>(sb, 0, 0, lane);
        vr[1] = lds_v<E>(sb, 0, 1, lane);
#pragma unroll
        for (int i = 0; i < kDv / 16; ++i) {
          const int d = i >> 1, kb = i & 1;
          const bf16x8 vop = widen_v(vr[i & 1]);
          if (i + 2 < kDv / 16) vr[i & 1] = lds_v<E>(sb, (i + 2) >> 1, (i + 2) & 1, lane);
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
    uint8_t *stg = lds + 2 * Tile<E>::kBytes + wave * Staging<E>::kWaveBytes;
    // output pointers are read where they are used (see kernarg_args): a
    // copy kept from the kernel's start would be reloaded from scratch after
    // the row stores, and that reload's wait would drain every store first
    const KernargArgs ka = kernarg_args();
    if (complete) {
      __bf16 *orow0 = (__bf16 *)ka->out + ((int64_t)b * a.M + mt * kTileRows + wave * kWaveRows) * kDv;
      store_rows<E>(oacc, inv, stg, orow0, nrows);
      if (mvalid && h == 0)
        ka->lse[(int64_t)b * a.M + mt * kTileRows + wave * kWaveRows + (fresh_lane_id() & 31)] =
            has ? lse2 * kLn2 : kNegInf;
    } else {
      // rows past M are never merged: no partial for them
      const int64_t prow0 = (w * kSlots + piece_slot(P.st_begin)) * kTileRows + wave * kWaveRows;
      if constexpr (E == 1) {
        // fp16 partial of o / kv_scale: a weighted mean of E4M3 values, so
        // |value| <= 448 and fp16 keeps 11 significant bits of it
        const float invr = has ? 1.0f / ltot : 0.f;
        store_rows<E>(oacc, invr, stg, (_Float16 *)ka->ws_o + prow0 * kDv, nrows);
      } else {
        store_rows<E>(oacc, inv, stg, (float *)ka->ws_o + prow0 * kDv, nrows);
      }
      if (mvalid && h == 0) ka->ws_lse2[prow0 + (fresh_lane_id() & 31)] = lse2;
    }
    if (!more) break;
    P = following;
  }
  if (bad) atomicOr(a.err, DCPMLA_ERR_PAGE_RANGE);
}

constexpr size_t kLdsLimit = 160 * 1024;   // gfx950 LDS per workgroup

template <int E, bool PartLds, bool QF8>
hipError_t launch_variant(const AttnArgs &a, int groups, size_t shmem, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    const size_t cap = PartLds ? kLdsLimit : 2 * Tile<E>::kBytes + Staging<E>::kBytes;
    const hipError_t e = hipFuncSetAttribute((const void *)attention_kernel<E, PartLds, QF8>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)cap);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((attention_kernel<E, PartLds, QF8>), dim3(groups), dim3(kThreads), shmem, stream, a);
  return hipGetLastError();
}

template <int E, bool QF8>
hipError_t launch_tile(AttnArgs a, int groups, hipStream_t stream) {
  const size_t tiles = 2 * Tile<E>::kBytes + Staging<E>::kBytes;
  const size_t part = (size_t)(4 * (int64_t)a.B + 2 + (int64_t)a.B * a.qlen) * 4;
  if (tiles + part <= kLdsLimit) {
    a.part_ints = (int)(part / 4);
    return launch_variant<E, true, QF8>(a, groups, tiles + part, stream);
  }
  a.part_ints = 0;
  return launch_variant<E, false, QF8>(a, groups, tiles, stream);
}

}  // namespace

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
  a.score_scale2 = softmax_scale * kv_scale * 1.44269504088896340736f;
  a.out_scale = kv_scale;
  const int64_t rows = (int64_t)g.batch * a.M;
  if (g.kv_dtype == DCPMLA_KV_FP8_E4M3) {
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
    if (g.q_format == DCPMLA_Q_FP8) return launch_tile<1, true>(a, groups, stream);
    return launch_tile<1, false>(a, groups, stream);
  }
  return launch_tile<2, false>(a, groups, stream);
}

}  // namespace dcpmla
