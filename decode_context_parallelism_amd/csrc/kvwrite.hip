// Interleaved KV write for one DCP rank.
//
// "Context Parallel Guide (PCP & DCP)" (ATOM docs): the cache is interleaved
// across the DCP group, token p living on rank (p // S) % W (--dcp-config,
// interleave_size); one virtual block id names, on every rank, that rank's
// own physical block of block_size rank-local tokens ("How it works" item 1);
// new-token KV is written through a slot mapping that holds -1 for tokens the
// rank does not own (item 2).  The rank-local index is
// (p // (S*W)) * S + p % S (interleave_size constraints).
#include "common.h"
#include "launch.h"

namespace dcpmla {

__global__ void __launch_bounds__(256) write_kv_kernel(
    int W, int S, int block_size, int max_blocks, int batch, int64_t num_blocks, int rank,
    int64_t num_tokens, int units_per_token, const int32_t *__restrict__ seq_ids,
    const int32_t *__restrict__ positions, const uint4 *__restrict__ latents,
    const int32_t *__restrict__ block_table, uint4 *__restrict__ pool,
    int32_t *__restrict__ slot_mapping, int32_t *__restrict__ err) {
  const int64_t n = num_tokens * units_per_token;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = u / units_per_token;
    const int part = (int)(u - t * units_per_token);
    const int b = seq_ids[t];
    const int p = positions[t];
    int64_t slot = -1;
    int e = 0;
    if (b < 0 || b >= batch || p < 0) {
      e = DCPMLA_ERR_TOKEN;
    } else if ((p / S) % W == rank) {
      const int64_t li = (int64_t)(p / (S * W)) * S + p % S;
      const int64_t vb = li / block_size;
      if (vb >= max_blocks) {
        e = DCPMLA_ERR_TABLE_CAPACITY;
      } else {
        const int32_t blk = block_table[(int64_t)b * max_blocks + vb];
        if (blk < 0 || (int64_t)blk >= num_blocks)
          e = DCPMLA_ERR_BLOCK_ID;
        else
          slot = (int64_t)blk * block_size + li % block_size;
      }
    }
    if (slot >= 0) pool[slot * units_per_token + part] = latents[t * units_per_token + part];
    if (part == 0) {
      slot_mapping[t] = slot >= 0 ? (int32_t)slot : -1;
      if (e) atomicOr(err, e);
    }
  }
}

hipError_t launch_write_kv(const dcpmla_geom &g, int rank, int64_t num_tokens,
                           const int32_t *seq_ids, const int32_t *positions, const void *latents,
                           const int32_t *block_table, void *kv_pool, int32_t *slot_mapping,
                           int32_t *err, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int elem = g.kv_dtype == DCPMLA_KV_FP8_E4M3 ? 1 : 2;
  const int units = kDqk * elem / 16;
  const int64_t n = num_tokens * units;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g.dcp_world,
                     g.interleave, g.block_size, g.max_blocks_per_seq, g.batch, g.num_blocks, rank,
                     num_tokens, units, seq_ids, positions, (const uint4 *)latents, block_table,
                     (uint4 *)kv_pool, slot_mapping, err);
  return hipGetLastError();
}

}  // namespace dcpmla
