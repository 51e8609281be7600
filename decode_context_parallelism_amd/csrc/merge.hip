// LSE merges: split-KV segments (base-2 statistics -> BF16 output plus
// natural-log LSE) and DCP ranks (natural-log LSE -> BF16 output).
//
// Segment merge: "[ROCm][MLA][DCP] Support causal multi-token verification"
// (vLLM PR #51705), "Implementation" item 3 and its commit message (decode
// LSE is natural-log; the segment merge converts the kernel's base-2
// statistics).  Rank merge: "Context Parallel Guide (PCP & DCP)",
// enable_project_before_merge (a per-(token, head) scalar weight and a
// cross-rank sum); an empty rank carries LSE = -inf and adds nothing.
//
// Layout of the work: one wave per output row, each lane owning 8 of the 512
// value dims (16-byte loads and stores), so a row is two fully coalesced
// 1 KiB (BF16) or 2 KiB (float) transactions per partial.
#include "common.h"
#include "launch.h"

namespace dcpmla {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a;
  const __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ inline uint4 pack_bf16x8(const float *v) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

__device__ inline void unpack_bf16x8(uint4 u, float *v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf16_to_f32(w[k] & 0xFFFFu);
    v[2 * k + 1] = bf16_to_f32(w[k] >> 16);
  }
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace

// Ranks are taken kRankBatch at a time: the batch's LSEs and rows are
// requested together and merged against a running maximum, so up to
// kRankBatch ranks cost one memory round trip.
constexpr int kRankBatch = 8;

__global__ void __launch_bounds__(256) merge_ranks_kernel(int W, int64_t rows,
                                                          const uint4 *__restrict__ out_ranks,
                                                          const float *__restrict__ lse_ranks,
                                                          uint4 *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float mx = kNegInf;
  float z = 0.f;
  for (int r0 = 0; r0 < W; r0 += kRankBatch) {
    float l[kRankBatch];
    float v[kRankBatch][8];
#pragma unroll
    for (int q = 0; q < kRankBatch; ++q) {
      // entries past W repeat the last rank (a valid address) and are dropped below
      const int r = r0 + q < W ? r0 + q : W - 1;
      l[q] = r0 + q < W ? lse_ranks[(int64_t)r * rows + row] : kNegInf;
      unpack_bf16x8(out_ranks[((int64_t)r * rows + row) * 64 + lane], v[q]);
    }
    float bm = kNegInf;
#pragma unroll
    for (int q = 0; q < kRankBatch; ++q) bm = fmaxf(bm, l[q]);
    if (bm > mx) {
      // rescale what was summed against the old maximum (nothing when it was -inf)
      const float c = mx > kNegInf ? fast_exp2((mx - bm) * kLog2e) : 0.f;
      z *= c;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= c;
      mx = bm;
    }
    if (mx > kNegInf) {
#pragma unroll
      for (int q = 0; q < kRankBatch; ++q) {
        // an empty rank (LSE = -inf) adds nothing
        const float w = l[q] > kNegInf ? fast_exp2((l[q] - mx) * kLog2e) : 0.f;
        z += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * v[q][e];
      }
    }
  }
  float L = kNegInf;
  if (mx > kNegInf) {
    const float inv = 1.f / z;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= inv;
    L = mx + fast_log2(z) * kLn2;
  }
  out[row * 64 + lane] = pack_bf16x8(acc);
  if (lane == 0) lse[row] = L;
}

__global__ void __launch_bounds__(256) merge_segments_dense_kernel(
    int64_t rows, int nseg, const float4 *__restrict__ o_seg, const float *__restrict__ lse2_seg,
    uint4 *__restrict__ out, float *__restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float *l2 = lse2_seg + row * nseg;
  float mx = kNegInf;
  for (int s = 0; s < nseg; ++s) mx = fmaxf(mx, l2[s]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float L = kNegInf;
  if (mx > kNegInf) {
    float z = 0.f;
    for (int s = 0; s < nseg; ++s) {
      const float l = l2[s];
      if (!(l > kNegInf)) continue;
      const float w = fast_exp2(l - mx);
      z += w;
      const float4 *src = o_seg + ((row * nseg + s) * kDv) / 4 + 2 * lane;
      const float4 a = src[0], b = src[1];
      acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
      acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
    }
    const float inv = 1.f / z;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= inv;
    L = (mx + fast_log2(z)) * kLn2;
  }
  out[row * 64 + lane] = pack_bf16x8(acc);
  if (lane == 0) lse[row] = L;
}

// Persistent layout: finish every (sequence, head-row tile) whose stages were
// split over several workgroups, and give sequences with no rank-local token
// their empty result.  Tiles finished inside one workgroup are left alone.
// One workgroup per (sequence, tile, group of 4 RPW rows), rows wave, wave + 4,
// ... of the group on each wave; the partials of a row are requested
// kMergeBatch at a time, their base-2 LSEs with them, and merged against a
// running maximum, so a row costs one dependent memory round trip per batch
// (no separate pass for the maximum).  Most items of a batch with many
// sequences finish inside one attention workgroup and their merge workgroups
// only read the partition and leave: past about as many workgroups as the
// chip holds at once, two rows per wave halve the grid, measured 15% faster
// on 32 sequences x 5 tiles and slower where every item is split.
constexpr int kMergeBatch = 8;
constexpr int kMergeGroupsResident = 2048;

// Partial loads: 8 value dims of one partial row for this lane.
__device__ inline void load_partial8(const float *row, int lane, float v[8]) {
  const float4 a = ((const float4 *)row)[2 * lane], b = ((const float4 *)row)[2 * lane + 1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ inline void load_partial8(const _Float16 *row, int lane, float v[8]) {
  typedef _Float16 half8v __attribute__((ext_vector_type(8)));
  const half8v h = __builtin_bit_cast(half8v, ((const uint4 *)row)[lane]);
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (float)h[k];
}

template <typename PT, int RPW>
__global__ void __launch_bounds__(256) merge_segments_kernel(
    int B, int qlen, int heads, int n_mt, int G, int kv_dtype, const int32_t *__restrict__ work,
    const PT *__restrict__ ws_o, const float *__restrict__ ws_lse2, const float *__restrict__ ws_scale,
    uint4 *__restrict__ out, float *__restrict__ lse) {
  constexpr int rows_per_group = 4 * RPW;
  constexpr int chunks = kTileRows / rows_per_group;
  const int chunk = blockIdx.x % chunks;
  const int bt = blockIdx.x / chunks;
  const int b = bt / n_mt;
  const int mt = bt - b * n_mt;
  const int M = qlen * heads;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t U = work[0];
  const int stages = work[work_stages_off(B) + b];
  const int row0 = mt * kTileRows + chunk * rows_per_group;   // first row of this chunk
  const int nrows = min(rows_per_group, M - row0);
  if (nrows <= 0) return;
  if (stages == 0) {
    // no rank-local token for the whole sequence: O = 0, LSE = -inf
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int rw = wave + 4 * j;
      if (rw >= nrows) break;
      const int64_t orow = (int64_t)b * M + row0 + rw;
      out[orow * 64 + lane] = make_uint4(0, 0, 0, 0);
      if (lane == 0) lse[orow] = kNegInf;
    }
    return;
  }
  // the teams holding this item's first and last stage (cost positions x0
  // and x0 + stages - 1 of the walk); when they differ, the tile's group in
  // the first of them wrote its share to its slot 1 and each later one to
  // its slot 0
  const Split sp = work_split(G, U, n_mt, B, kv_dtype);
  const int item = mt / sp.tm, tpos = mt - item * sp.tm;
  const int64_t x0 = seq_cost(work[work_unit_base_off() + b] / sp.tm, sp.n_items, b, sp.pc) +
                     (int64_t)item * (stages + sp.pc) + sp.pc;
  const int64_t t0 = cost_group(x0, sp.C, sp.T);
  const int64_t t1 = cost_group(x0 + stages - 1, sp.C, sp.T);
  if (t0 == t1) return;   // finished inside one workgroup
  const int n = (int)(t1 - t0 + 1);
  auto src_of = [&](int k) {
    return ((t0 + k) * sp.tm + tpos) * kSlots + (k == 0 ? piece_slot(0) : piece_slot(1));
  };
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int rw = wave + 4 * j;
    if (rw >= nrows) break;
    const int pr0 = chunk * rows_per_group + rw;   // row index inside the tile (partial rows)
    // One pass with a running maximum: each batch's base-2 LSEs and partial
    // rows are requested together, the sums are rescaled when the maximum
    // moves, so an item split into at most kMergeBatch parts costs one memory
    // round trip.
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float mx = kNegInf;
    float z = 0.f;
    for (int k = 0; k < n; k += kMergeBatch) {
      float l[kMergeBatch];
      float v[kMergeBatch][8];
#pragma unroll
      for (int q = 0; q < kMergeBatch; ++q) {
        // entries past n repeat the last partial and are dropped below (a valid address)
        const int kk = k + q < n ? k + q : n - 1;
        const int64_t pr = src_of(kk) * kTileRows + pr0;
        l[q] = k + q < n ? ws_lse2[pr] : kNegInf;
        load_partial8(ws_o + pr * kDv, lane, v[q]);
      }
      float bm = kNegInf;
#pragma unroll
      for (int q = 0; q < kMergeBatch; ++q) bm = fmaxf(bm, l[q]);
      if (bm > mx) {
        // rescale what was summed against the old maximum (nothing when it was -inf)
        const float c = mx > kNegInf ? fast_exp2(mx - bm) : 0.f;
        z *= c;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= c;
        mx = bm;
      }
      if (mx > kNegInf) {
#pragma unroll
        for (int q = 0; q < kMergeBatch; ++q) {
          const float wgt = l[q] > kNegInf ? fast_exp2(l[q] - mx) : 0.f;
          z += wgt;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += wgt * v[q][e];
        }
      }
    }
    float L = kNegInf;
    if (mx > kNegInf) {
      // fp16 partials carry o / kv_scale
      const float inv = (sizeof(PT) == 2 ? *ws_scale : 1.f) / z;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] *= inv;
      L = (mx + fast_log2(z)) * kLn2;
    }
    const int64_t orow = (int64_t)b * M + row0 + rw;
    out[orow * 64 + lane] = pack_bf16x8(acc);
    if (lane == 0) lse[orow] = L;
  }
}

hipError_t launch_merge_ranks(int world, int64_t rows, const void *out_ranks,
                              const float *lse_ranks, void *out, float *lse, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(merge_ranks_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, world, rows,
                     (const uint4 *)out_ranks, lse_ranks, (uint4 *)out, lse);
  return hipGetLastError();
}

hipError_t launch_merge_segments_dense(int64_t rows, int nseg, const float *o_seg,
                                       const float *lse2_seg, void *out, float *lse,
                                       hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(merge_segments_dense_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     rows, nseg, (const float4 *)o_seg, lse2_seg, (uint4 *)out, lse);
  return hipGetLastError();
}

template <int RPW>
hipError_t launch_merge_segments_rpw(const dcpmla_geom &g, int groups, const dcpmla_meta &m, int n_mt,
                                     int64_t items, const void *workspace, void *out_rank,
                                     float *lse_rank, hipStream_t stream) {
  const float *ws = (const float *)workspace;
  const dim3 grid((unsigned)(items * (kTileRows / (4 * RPW))));
  if (g.kv_dtype == DCPMLA_KV_FP8_E4M3) {
    hipLaunchKernelGGL((merge_segments_kernel<_Float16, RPW>), grid, dim3(256), 0, stream, g.batch, g.qlen,
                       g.num_heads, n_mt, groups, g.kv_dtype, m.work, (const _Float16 *)workspace,
                       ws + ws_o_floats(groups), ws + ws_scale_off(groups), (uint4 *)out_rank, lse_rank);
  } else {
    hipLaunchKernelGGL((merge_segments_kernel<float, RPW>), grid, dim3(256), 0, stream, g.batch, g.qlen,
                       g.num_heads, n_mt, groups, g.kv_dtype, m.work, ws, ws + ws_o_floats(groups),
                       ws + ws_scale_off(groups), (uint4 *)out_rank, lse_rank);
  }
  return hipGetLastError();
}

hipError_t launch_merge_segments(const dcpmla_geom &g, int groups, const dcpmla_meta &m,
                                 const void *workspace, void *out_rank, float *lse_rank,
                                 hipStream_t stream) {
  const int n_mt = n_mtiles(g.qlen, g.num_heads);
  const int64_t items = (int64_t)g.batch * n_mt;
  if (items * (kTileRows / 4) > kMergeGroupsResident)
    return launch_merge_segments_rpw<2>(g, groups, m, n_mt, items, workspace, out_rank, lse_rank, stream);
  return launch_merge_segments_rpw<1>(g, groups, m, n_mt, items, workspace, out_rank, lse_rank, stream);
}

}  // namespace dcpmla
