// Verify-view builder: per-row causal boundary, rank-local length, bounded
// subpage expansion, and the split-KV work partition.
//
// "[ROCm][MLA][DCP] Support causal multi-token verification" (vLLM PR
// #51705), "Implementation" items 1, 2 and 5: each verification row gets its
// own global causal boundary mapped to a rank-local KV length; physical blocks
// are expanded into bounded subpages; row metadata lives in stable buffers
// sized by a static bound.  The length formula is the one computed per query
// in "[Spec decode] Support Kimi-K3 DCP with DSpark" (vLLM PR #52188), review
// thread.
#include "common.h"
#include "launch.h"

namespace dcpmla {

namespace {

// Row i of sequence b: its global boundary, rank-local length and subpage
// count, with the capacity clamps (before any block-id check).
struct RowGeom {
  int64_t len;
  int np;
  int err;
};
__device__ inline RowGeom row_geometry(int64_t ctx, int i, int W, int S, int qlen, int P, int ppb,
                                       int max_blocks, int max_local_pages, int rank, int block_rows) {
  int e = 0;
  // global boundary of row i: causal verify, or the whole cache for a
  // bidirectional draft block
  int64_t g = block_rows ? ctx : ctx - qlen + 1 + i;
  if (ctx < qlen) e |= DCPMLA_ERR_CTX_LT_QLEN;
  if (g < 0) g = 0;
  const int64_t span = (int64_t)W * S;
  int64_t rem = g % span - (int64_t)rank * S;
  rem = rem < 0 ? 0 : (rem > S ? S : rem);
  int64_t len = (g / span) * S + rem;    // rank-local tokens visible to the row
  int64_t np = (len + P - 1) / P;
  const int64_t cap = (int64_t)max_blocks * ppb;
  if (np > cap) { np = cap; e |= DCPMLA_ERR_TABLE_CAPACITY; }
  if (np > max_local_pages) { np = max_local_pages; e |= DCPMLA_ERR_LOCAL_PAGES; }
  if (len > np * P) len = np * P;
  return RowGeom{len, (int)np, e};
}

}  // namespace

__global__ void __launch_bounds__(256) meta_rows_kernel(
    int W, int S, int block_size, int qlen, int max_blocks, int max_local_pages,
    int64_t num_blocks, int rank, int block_rows, const int32_t *__restrict__ ctx_lens,
    const int32_t *__restrict__ block_table, int32_t *__restrict__ row_len,
    int32_t *__restrict__ page_table, int32_t *__restrict__ last_len, int32_t *__restrict__ err) {
  const int row = blockIdx.x;
  const int b = row / qlen;
  const int i = row - b * qlen;
  const int P = subpage_size(block_size);
  const int ppb = block_size / P;
  __shared__ int s_np, s_err, s_first_bad;
  __shared__ int64_t s_len;
  if (threadIdx.x == 0) {
    const RowGeom r = row_geometry(ctx_lens[b], i, W, S, qlen, P, ppb, max_blocks, max_local_pages,
                                   rank, block_rows);
    s_np = r.np;
    s_len = r.len;
    s_err = r.err;
    s_first_bad = r.np;
  }
  __syncthreads();
  int np = s_np;
  const int32_t *bt = block_table + (int64_t)b * max_blocks;
  // every block id the row uses must name a block of the pool; the load is
  // bounded by the row's own page count, so unused (poisoned) entries are
  // never read
  for (int j = threadIdx.x; j < np; j += blockDim.x) {
    const int32_t blk = bt[j / ppb];
    if (blk < 0 || (int64_t)blk >= num_blocks) atomicMin(&s_first_bad, j);
  }
  __syncthreads();
  const int first_bad = s_first_bad;
  if (first_bad < np) np = first_bad;
  int64_t len = s_len;
  if (len > (int64_t)np * P) len = (int64_t)np * P;
  int32_t *pt = page_table + (int64_t)row * max_local_pages;
  for (int j = threadIdx.x; j < max_local_pages; j += blockDim.x) {
    int32_t v = -1;
    if (j < np) v = bt[j / ppb] * ppb + (j % ppb);
    pt[j] = v;
  }
  if (threadIdx.x == 0) {
    row_len[row] = (int32_t)len;
    last_len[row] = np ? (int32_t)(len - (int64_t)(np - 1) * P) : 0;
    const int e = s_err | (first_bad < s_np ? DCPMLA_ERR_BLOCK_ID : 0);
    if (e) atomicOr(err, e);
  }
}

// One workgroup: longest row per sequence, stages, and the unit prefix.
__global__ void __launch_bounds__(256) meta_work_kernel(int B, int qlen, int n_mt, int stage,
                                                        const int32_t *__restrict__ row_len,
                                                        int32_t *__restrict__ work) {
  __shared__ int s_scan[256];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int units = 0;
    if (b < B) {
      int lm = 0, lrow = b * qlen + qlen - 1;
      for (int i = 0; i < qlen; ++i) {
        const int v = row_len[b * qlen + i];
        if (v > lm) { lm = v; lrow = b * qlen + i; }
      }
      const int st = (lm + stage - 1) / stage;
      work[work_lmax_off(B) + b] = lm;
      work[work_lrow_off(B) + b] = lrow;
      work[work_stages_off(B) + b] = st;
      units = st * n_mt;
    }
    s_scan[tid] = units;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    if (b < B) work[work_unit_base_off() + b] = s_carry + s_scan[tid] - units;
    __syncthreads();
    if (tid == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  if (tid == 0) {
    work[work_unit_base_off() + B] = s_carry;
    work[0] = s_carry;
  }
  for (int i = tid; i < kZeroInts; i += 256) work[work_zero_off(B) + i] = 0;
}

// Small verify views (rows * max_local_pages <= kSmallEntries, rows and
// sequences <= kSmallThreads): the same per-row steps and the partition in
// one workgroup, so the view costs one launch instead of two.
constexpr int kSmallThreads = 1024;
constexpr int kSmallEntries = 8192;

__global__ void __launch_bounds__(kSmallThreads) meta_small_kernel(
    int W, int S, int block_size, int qlen, int max_blocks, int max_local_pages, int64_t num_blocks,
    int rank, int block_rows, int B, int n_mt, int stage, const int32_t *__restrict__ ctx_lens,
    const int32_t *__restrict__ block_table, int32_t *__restrict__ row_len,
    int32_t *__restrict__ page_table, int32_t *__restrict__ last_len, int32_t *__restrict__ err,
    int32_t *__restrict__ work) {
  constexpr int kWaves = kSmallThreads / 64;
  constexpr int kPerThread = kSmallEntries / kSmallThreads;
  __shared__ int s_np[kSmallThreads], s_len[kSmallThreads], s_first_bad[kSmallThreads];
  __shared__ int s_row_err[kSmallThreads];
  __shared__ int s_wave_sum[kWaves];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int rows = B * qlen;
  const int n_entries = rows * max_local_pages;
  const int P = subpage_size(block_size);
  const int ppb = block_size / P;
  // per-row boundary, length and page count (one thread per row)
  if (tid < rows) {
    const int b = tid / qlen;
    const RowGeom r = row_geometry(ctx_lens[b], tid - b * qlen, W, S, qlen, P, ppb, max_blocks,
                                   max_local_pages, rank, block_rows);
    s_np[tid] = r.np;
    s_len[tid] = (int)r.len;   // <= max_local_pages * 128
    s_first_bad[tid] = r.np;
    s_row_err[tid] = r.err;
  }
  if (tid == 0) s_err = 0;
  __syncthreads();
  // block ids each row uses, bounded by its page count; each thread keeps
  // the ids of its entries for the page table below (one read of the table)
  int32_t blk[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int idx = tid + k * kSmallThreads;
    blk[k] = -1;
    if (idx < n_entries) {
      const int row = idx / max_local_pages, j = idx - row * max_local_pages;
      if (j < s_np[row]) {
        blk[k] = block_table[(int64_t)(row / qlen) * max_blocks + j / ppb];
        if (blk[k] < 0 || (int64_t)blk[k] >= num_blocks) atomicMin(&s_first_bad[row], j);
      }
    }
  }
  __syncthreads();
  if (tid < rows) {
    int np = s_np[tid];
    int e = s_row_err[tid];
    if (s_first_bad[tid] < np) {
      np = s_first_bad[tid];
      e |= DCPMLA_ERR_BLOCK_ID;
    }
    if (e) atomicOr(&s_err, e);
    const int len = min(s_len[tid], np * P);
    s_np[tid] = np;
    s_len[tid] = len;
    row_len[tid] = len;
    last_len[tid] = np ? len - (np - 1) * P : 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int idx = tid + k * kSmallThreads;
    if (idx < n_entries) {
      const int row = idx / max_local_pages, j = idx - row * max_local_pages;
      page_table[idx] = j < s_np[row] ? blk[k] * ppb + (j % ppb) : -1;
    }
  }
  // the work partition (as meta_work_kernel), one thread per sequence
  int units = 0;
  if (tid < B) {
    int lm = 0, lrow = tid * qlen + qlen - 1;
    for (int i = 0; i < qlen; ++i) {
      const int v = s_len[tid * qlen + i];
      if (v > lm) { lm = v; lrow = tid * qlen + i; }
    }
    const int st = (lm + stage - 1) / stage;
    work[work_lmax_off(B) + tid] = lm;
    work[work_lrow_off(B) + tid] = lrow;
    work[work_stages_off(B) + tid] = st;
    units = st * n_mt;
  }
  // prefix sum of the units: inclusive within each wave by shuffles, then
  // the waves' totals in order
  int incl = units;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wave_sum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int v = s_wave_sum[i];
    before += i < wv ? v : 0;
    total += v;
  }
  if (tid < B) work[work_unit_base_off() + tid] = before + incl - units;
  if (tid == 0) {
    work[work_unit_base_off() + B] = total;
    work[0] = total;
    if (s_err) atomicOr(err, s_err);
  }
  for (int i = tid; i < kZeroInts; i += kSmallThreads) work[work_zero_off(B) + i] = 0;
}

hipError_t launch_build_metadata(const dcpmla_geom &g, int rank, const int32_t *ctx_lens,
                                 const int32_t *block_table, const dcpmla_meta &m,
                                 hipStream_t stream) {
  const int rows = g.batch * g.qlen;
  if (rows <= kSmallThreads && (int64_t)rows * g.max_local_pages <= kSmallEntries) {
    hipLaunchKernelGGL(meta_small_kernel, dim3(1), dim3(kSmallThreads), 0, stream, g.dcp_world,
                       g.interleave, g.block_size, g.qlen, g.max_blocks_per_seq, g.max_local_pages,
                       g.num_blocks, rank, g.row_boundary == DCPMLA_BOUNDARY_BLOCK ? 1 : 0, g.batch,
                       n_mtiles(g.qlen, g.num_heads), stage_tokens(g.kv_dtype), ctx_lens, block_table,
                       m.row_local_len,
                       m.page_table, m.last_page_len, m.err, m.work);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(meta_rows_kernel, dim3(rows), dim3(256), 0, stream, g.dcp_world,
                     g.interleave, g.block_size, g.qlen, g.max_blocks_per_seq, g.max_local_pages,
                     g.num_blocks, rank, g.row_boundary == DCPMLA_BOUNDARY_BLOCK ? 1 : 0, ctx_lens,
                     block_table, m.row_local_len, m.page_table,
                     m.last_page_len, m.err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(meta_work_kernel, dim3(1), dim3(256), 0, stream, g.batch, g.qlen,
                     n_mtiles(g.qlen, g.num_heads), stage_tokens(g.kv_dtype), m.row_local_len, m.work);
  return hipGetLastError();
}

}  // namespace dcpmla
