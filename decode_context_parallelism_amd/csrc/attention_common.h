// Device code shared by the segmented attention kernels (BF16 cache:
// attention.hip; FP8 cache: attention_fp8.hip).  Internal, not part of the ABI.
#pragma once

#include <mutex>

#include "common.h"

namespace dcpmla {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
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
  int kv_dtype;              // DCPMLA_KV_*: fixes the stage size and the partition's piece cost
  float score_scale2;        // softmax_scale * kv_scale * log2(e)
  float out_scale;           // kv_scale
};
// Kernels take AttnArgs by value as their only argument, so it starts at
// offset 0 of the kernel-argument segment (read through kernarg_args below).
static_assert(sizeof(AttnArgs) % 8 == 0, "AttnArgs layout");

// This lane's index in the wave, read from the hardware at each call (a
// volatile asm the compiler can neither hoist nor keep live across loops:
// recomputing it is cheaper than a register held through the stage loop).
__device__ inline int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The kernel's argument block as it sits in the kernel-argument segment.
// Reading a field through this pointer is a scalar load; the empty asm makes
// each call a fresh pointer, so the compiler re-reads the field where it is
// used instead of holding it in registers across the kernel.
typedef const __attribute__((address_space(4))) AttnArgs *KernargArgs;
__device__ inline KernargArgs kernarg_args() {
  KernargArgs p = (KernargArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// Accumulator layout: register r of a 32x32 accumulator in lane half h holds
// row 8*(r/4) + 4*h + r%4 of the MFMA output tile, so in a score tile it
// holds that token of the tile.
//
// LDS row slot of tile token t (and, being an involution -- it swaps bits 2
// and 3 -- the token of slot t).  The p.v operand of lane half h gathers the
// eight tokens {4h..4h+3, 8+4h..8+4h+3} (+16 for the second token half);
// storing those eight rows in consecutive slots 8h..8h+7 makes each 16-lane
// transposing read touch every bank exactly once.
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

__device__ inline int8v cat8(uint4 a, uint4 b) {
  int8v r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
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
// all banks.  Waves never share an area, so no barrier is needed.  PB is the
// widest element stored (2: BF16 / fp16; 4: float).
template <int PB>
struct Staging {
  static constexpr int kPassDims = 128;
  static constexpr int kRowBytes = kPassDims * PB + 16;
  static constexpr int kWaveBytes = kWaveRows * kRowBytes;
  static constexpr int kBytes = kWaves * kWaveBytes;
};

// rows[r * kDv + c] = T(acc(row r, dim c) * sc) for rows r < nrows; T is
// __bf16, _Float16 or float.  The row stores are raw buffer stores whose
// resource covers only the nrows valid rows, so rows past the end are
// dropped by the range check instead of being branched around: a branch per
// store makes the compiler keep values across it in scratch, and each
// reload's wait would then also wait for every store issued before it.
template <int PB, typename T>
__device__ inline void store_rows(const floatx16 (&acc)[kDv / 32], float sc, uint8_t *stg, T *rows,
                                  int nrows) {
  constexpr int kRow = Staging<PB>::kRowBytes;
  constexpr int kSegBytes = Staging<PB>::kPassDims * (int)sizeof(T);
  constexpr int kLanesPerRow = kSegBytes / 16;
  constexpr int kRowsPerRead = 64 / kLanesPerRow;
  constexpr int kRowBytes = kDv * (int)sizeof(T);
  static_assert(sizeof(T) <= PB, "staging row too narrow");
  // addresses derived from the lane are recomputed per call, not hoisted
  // out of the piece loop (where they would stay live through the stages)
  const int lane = fresh_lane_id();
  const int l32 = lane & 31, h = lane >> 5;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(rows, (short)0, nrows > 0 ? nrows * kRowBytes : 0, kRawBufferFlags);
  const int rlane = lane / kLanesPerRow, c = lane % kLanesPerRow;
#pragma unroll
  for (int pass = 0; pass < kDv / Staging<PB>::kPassDims; ++pass) {
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

// ---------------------------------------------------------------- work walk
//
// The group's units [lo, hi) of the cost partition (common.h) are walked as
// one stream of (piece, stage) cursors.  A piece is one (sequence, tile) and
// the run of its stages this group owns.

struct Cursor {
  int b, mt, s;          // sequence, head-row tile, stage
  int st_begin, st_end;  // this group's stages of the piece
  int stages;            // stages of sequence b
  int lmax, lrow;        // b's longest rank-local row length and the row that has it
};

// Partition values are the same for the whole workgroup: they are read from
// the LDS copy (PartLds) or global memory and kept in scalar registers.
template <bool PartLds>
struct Walk {
  const int32_t *work;       // global partition
  const int32_t *part;       // its LDS copy (PartLds), then the row lengths
  const int32_t *row_len;    // global row lengths
  int B, n_mt, nwork;        // n_mt: items per sequence in this walk (Split::n_items)
  int tm;                    // groups per team: the partition's unit bases / tm are the walk's
  int64_t U, C, pc, hi;

  __device__ int32_t at(int i) const {
    if constexpr (PartLds) return __builtin_amdgcn_readfirstlane(part[i]);
    else return __builtin_amdgcn_readfirstlane(work[i]);
  }
  __device__ int64_t base_at(int b) const { return (int64_t)at(work_unit_base_off() + b) / tm; }
  __device__ int32_t row_len_at(int i) const {
    if constexpr (PartLds) return part[nwork + i];
    else return row_len[i];
  }
  // units whose cost position is below x (the unit index at cost x)
  __device__ int64_t units_before(int64_t x) const {
    if (x >= C) return U;
    int blo = 0, bhi = B;   // seq_cost(blo) <= x < seq_cost(bhi)
    while (bhi - blo > 1) {
      const int mid = (blo + bhi) >> 1;
      if (seq_cost(base_at(mid), n_mt, mid, pc) <= x) blo = mid; else bhi = mid;
    }
    const int64_t base = base_at(blo);
    const int64_t st = at(work_stages_off(B) + blo);
    const int64_t rem = x - seq_cost(base, n_mt, blo, pc);
    const int64_t mt = rem / (st + pc);
    const int64_t off = rem - mt * (st + pc) - pc;
    return base + mt * st + (off > 0 ? off : 0);
  }
  // per-sequence values, read once when a cursor reaches a sequence (not per stage)
  __device__ void enter_seq(Cursor &c) const {
    c.stages = at(work_stages_off(B) + c.b);
    c.lmax = at(work_lmax_off(B) + c.b);
    c.lrow = at(work_lrow_off(B) + c.b);
  }
  __device__ Cursor locate(int64_t u) const {
    int blo = 0, bhi = B;   // unit_base[blo] <= u < unit_base[bhi]
    while (bhi - blo > 1) {
      const int mid = (blo + bhi) >> 1;
      if (base_at(mid) <= u) blo = mid; else bhi = mid;
    }
    Cursor c;
    c.b = blo;
    enter_seq(c);
    const int64_t rem = u - base_at(blo);
    c.mt = (int)(rem / c.stages);
    c.s = (int)(rem - (int64_t)c.mt * c.stages);
    c.st_begin = c.s;
    c.st_end = (int)min((int64_t)c.stages, c.s + (hi - u));
    return c;
  }
  // cursor of unit u + 1 from that of unit u (u + 1 < hi)
  __device__ Cursor advance(Cursor c, int64_t u_next) const {
    if (++c.s < c.st_end) return c;
    if (++c.mt >= n_mt) {
      c.mt = 0;
      do { ++c.b; } while (at(work_stages_off(B) + c.b) == 0);
      enter_seq(c);
    }
    c.s = 0;
    c.st_begin = 0;
    c.st_end = (int)min((int64_t)c.stages, hi - u_next);
    return c;
  }
};

// Host side: runs f on the caller's current device until it succeeds once
// there (per-device kernel attributes such as the dynamic-LDS cap).
struct DeviceOnce {
  static constexpr int kMaxDevices = 64;
  std::mutex mu;
  bool done[kMaxDevices] = {};
  template <class F>
  hipError_t run(F f) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return f();
    std::lock_guard<std::mutex> lock(mu);
    if (done[dev]) return hipSuccess;
    e = f();
    if (e == hipSuccess) done[dev] = true;
    return e;
  }
};

}  // namespace attn

// The two kernel families' launchers (attention.hip, attention_fp8.hip).
hipError_t launch_attention_bf16(const attn::AttnArgs &a, int groups, hipStream_t stream);
hipError_t launch_attention_fp8(const attn::AttnArgs &a, int groups, bool q_fp8, bool p_fp8,
                                hipStream_t stream);

}  // namespace dcpmla
