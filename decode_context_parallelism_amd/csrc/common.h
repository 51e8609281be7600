// Internal definitions shared by the dcpmla HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcpmla.h"

namespace dcpmla {

constexpr int kDqk = 576;          // 512 latent + 64 rope
constexpr int kDv = 512;
constexpr int kRopeDims = kDqk - kDv;
constexpr int kStageTokens = 32;   // tokens per LDS stage with a BF16 cache (one 32x32 score tile)
constexpr int kStageTokensFp8 = 64;  // with an FP8 cache: two score tiles, one K = 64 product of p.v
constexpr int kWaveRows = 32;      // head-rows (M) per wave
constexpr int kWaves = 4;          // waves per attention workgroup
constexpr int kTileRows = kWaveRows * kWaves;  // head-rows per workgroup (M tile)
constexpr int kThreads = kWaves * 64;
constexpr int kSlots = 2;          // partial slots per persistent workgroup

// Stage size by cache format: the unit of the work partition below.
__host__ __device__ inline int stage_tokens(int kv_dtype) {
  return kv_dtype == DCPMLA_KV_FP8_E4M3 ? kStageTokensFp8 : kStageTokens;
}

// Work buffer layout (int32): [0] total units U; [1 .. B+1] unit_base[b]
// (prefix of n_mtiles * stages over sequences, unit_base[B] = U);
// [B+2 .. 2B+2) stages[b]; [2B+2 .. 3B+2) longest rank-local row length lmax[b];
// [3B+2 .. 4B+2) the verify row (b*qlen + i) that has that length.  A unit is
// one stage (stage_tokens(kv_dtype) tokens) of one (sequence, head-row tile).
// Past the partition, a zero row of kZeroInts int32 (one 576-element latent
// row in either cache format) that attention reads for tokens outside a
// sequence; the builder rewrites it with every forward.
constexpr int kZeroInts = kDqk * 2 / 4;
__host__ __device__ inline int64_t work_zero_off(int batch) { return ((4 * (int64_t)batch + 2 + 63) / 64) * 64; }
__host__ __device__ inline int64_t work_ints(int batch) { return work_zero_off(batch) + kZeroInts; }
__host__ __device__ inline int work_unit_base_off() { return 1; }
__host__ __device__ inline int work_stages_off(int batch) { return batch + 2; }
__host__ __device__ inline int work_lmax_off(int batch) { return 2 * batch + 2; }
__host__ __device__ inline int work_lrow_off(int batch) { return 3 * batch + 2; }

__host__ __device__ inline int subpage_size(int block_size) {
  int low = block_size & (-block_size);
  return low < 128 ? low : 128;
}

__host__ __device__ inline int n_mtiles(int qlen, int heads) {
  int m = qlen * heads;
  return (m + kTileRows - 1) / kTileRows;
}

// Workspace: o partials [groups][kSlots][kTileRows][kDv], then lse2 partials
// [groups][kSlots][kTileRows] float, then the partials' scale (one float,
// padded to 16 bytes).  With an FP8 cache the o partials are fp16 values of
// o / kv_scale (bounded by the E4M3 maximum 448) and the scale is kv_scale;
// with a BF16 cache they are float values of o and the scale is unused.
__host__ __device__ inline int64_t ws_o_floats(int groups) {
  return (int64_t)groups * kSlots * kTileRows * kDv;
}
__host__ __device__ inline int64_t ws_scale_off(int groups) {
  return ws_o_floats(groups) + (int64_t)groups * kSlots * kTileRows;
}
__host__ __device__ inline int64_t ws_bytes(int groups) { return (ws_scale_off(groups) + 4) * 4; }

// Then (256-byte aligned) the split query of an FP8-cache launch, q =
// (hi + lo) * 2^-k with 576 E4M3 codes hi and 576 codes lo per head-row,
// then one float 2^-k per head-row.
//
// The codes are tiled for the attention kernel's operand loads: rows go in
// blocks of 32 (block n holds rows 32n .. 32n + 31), and a block is 36
// chunks of 1 KiB.  Chunk c = 4t + 2 term + half (t < 9 the 64-dim step,
// term 0 = hi, 1 = lo) holds, at bytes 16 (32 g + i) .. +15, the 16 codes of
// row 32n + i, that term, dims 64t + 32g + 16 half .. +15 (g = 0, 1): the
// bytes lane 32g + i of a wave needs for that step, so each of the wave's
// query loads reads one contiguous KiB.  The last block is padded to 32
// rows.
constexpr int kQSplitRow = 2 * kDqk;                             // bytes per head-row
constexpr int kQSplitBlockRows = 32;
constexpr int kQSplitChunk = 1024;
constexpr int kQSplitBlock = kQSplitBlockRows * kQSplitRow;      // 36 chunks
__host__ __device__ inline int64_t qsplit_bytes(int64_t rows) {
  return (rows + kQSplitBlockRows - 1) / kQSplitBlockRows * kQSplitBlock;
}
// byte offset of chunk c's 16 bytes for row `row`, lane half g
__host__ __device__ inline int64_t qsplit_off(int64_t row, int c, int g) {
  return (row / kQSplitBlockRows) * kQSplitBlock + (int64_t)c * kQSplitChunk +
         (kQSplitBlockRows * g + row % kQSplitBlockRows) * 16;
}
__host__ __device__ inline int64_t ws_qsplit_off(int groups) { return ((ws_bytes(groups) + 255) / 256) * 256; }
__host__ __device__ inline int64_t ws_qscale_off(int groups, int64_t rows) {
  return ws_qsplit_off(groups) + qsplit_bytes(rows);
}
__host__ __device__ inline int64_t ws_total_bytes(int groups, int64_t rows) {
  return ws_qscale_off(groups, rows) + rows * 4;
}

// Workgroups that actually take work: every one gets at least about
// min_units(kv_dtype) stages (128 tokens), because each split costs a partial
// of 128 rows x 512 values (written here, read back by the segment merge) and
// a reload of the tile's query rows.  Four 32-token stages keep every compute
// unit busy on the small verify workload (about 1,200 stages per rank) and
// were measured faster there than eight.
__host__ __device__ inline int64_t min_units(int kv_dtype) {
  return kv_dtype == DCPMLA_KV_FP8_E4M3 ? 2 : 4;
}

// Scheduling cost.  Besides its stages, every (sequence, head-row tile) item
// costs piece_cost(kv_dtype) stage-equivalents for its query load and output
// stores, which dominate when sequences are short.  Measured, a piece's query
// load and output stores take about 16-18k cycles against about 4k per
// 32-token stage of the BF16-operand loop (5 measured best over the five
// workloads, 6 and 4 close), and about 4.5k per 64-token stage of the FP8 loop
// (3).  Every split piece pays them while the axis below charges them once per
// item.  Items are laid out on a cost axis in (sequence, tile) order, each as
// pc = piece_cost of overhead followed by its stages: item (b, mt) starts at
//   item_cost(b, mt) = unit_base[b] + pc * n_mt * b + mt * (stages[b] + pc)
// and its stage s sits at item_cost + pc + s.  Workgroup w of G owns the
// units whose cost position lies in [w C / G, (w + 1) C / G) with
// C = U + pc * n_mt * B.  Every group's cost range is non-empty (G <= U <= C),
// but it may hold only overhead and so no unit.
__host__ __device__ inline int64_t piece_cost(int kv_dtype) {
  return kv_dtype == DCPMLA_KV_FP8_E4M3 ? 3 : 5;
}
__host__ __device__ inline int64_t total_cost(int64_t U, int n_mt, int batch, int64_t pc) {
  return U + pc * n_mt * (int64_t)batch;
}
__host__ __device__ inline int64_t seq_cost(int64_t unit_base_b, int n_mt, int b, int64_t pc) {
  return unit_base_b + pc * n_mt * (int64_t)b;
}
// Head-row tiles run in teams: tm = n_mt consecutive logical groups (which
// share an XCD) walk the same columns -- (sequence, stage) -- in step, group
// t * tm + p taking tile p of each, so a stage's KV pages come from HBM once
// and the team's other tiles find them in that XCD's L2.  With fewer groups
// than tiles, tm = 1 and each group walks (sequence, tile, stage) alone.  The
// walk then sees n_mt / tm items per sequence of `stages` columns each; its
// unit bases are the partition's unit bases divided by tm.
struct Split {
  int tm;           // groups per team
  int n_items;      // items per sequence in a team's walk
  int64_t T;        // teams that take work
  int64_t cols;     // columns in the walk
  int64_t pc;       // cost of a piece's query load and output
  int64_t C;        // total cost of the walk
};
__host__ __device__ inline Split work_split(int64_t launched, int64_t U, int n_mt, int batch, int kv_dtype) {
  Split s;
  s.tm = launched >= n_mt ? n_mt : 1;
  s.n_items = n_mt / s.tm;
  s.cols = U / s.tm;
  const int64_t mu = min_units(kv_dtype);
  int64_t t = (s.cols + mu - 1) / mu;
  if (t < 1) t = 1;
  const int64_t tmax = launched / s.tm;
  s.T = t < tmax ? t : tmax;
  s.pc = piece_cost(kv_dtype);
  s.C = total_cost(s.cols, s.n_items, batch, s.pc);
  return s;
}
__host__ __device__ inline int64_t group_cost_lo(int64_t w, int64_t C, int64_t G) { return (w * C) / G; }
// the group whose cost range holds position x (0 <= x < C)
__host__ __device__ inline int64_t cost_group(int64_t x, int64_t C, int64_t G) { return ((x + 1) * G - 1) / C; }
// Partial slots: a piece that starts inside its item is its group's first
// piece (slot 0); a split piece that starts at the item's first stage ends
// inside the item and so is its group's last piece (slot 1).
__host__ __device__ inline int piece_slot(int first_stage) { return first_stage > 0 ? 0 : 1; }

// The dispatcher places workgroup i on XCD i % 8.  Logical group numbers
// (which fix the unit range) are handed out so that each XCD runs one
// contiguous range of them: neighbouring ranges share a sequence's query
// rows and KV pages, which then stay in that XCD's L2.  A bijection on
// [0, G) for workgroups i < G.
constexpr int64_t kXcds = 8;
__host__ __device__ inline int64_t xcd_group(int64_t i, int64_t G) {
  const int64_t x = i % kXcds, k = i / kXcds;
  const int64_t q = G / kXcds, r = G % kXcds;
  return x * q + (x < r ? x : r) + k;
}

}  // namespace dcpmla
