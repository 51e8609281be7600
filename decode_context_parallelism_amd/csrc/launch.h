// Internal launchers, one per kernel family (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "dcpmla.h"

namespace dcpmla {

hipError_t launch_build_metadata(const dcpmla_geom &g, int rank, const int32_t *ctx_lens,
                                 const int32_t *block_table, const dcpmla_meta &m,
                                 hipStream_t stream);

hipError_t launch_write_kv(const dcpmla_geom &g, int rank, int64_t num_tokens,
                           const int32_t *seq_ids, const int32_t *positions, const void *latents,
                           const int32_t *block_table, void *kv_pool, int32_t *slot_mapping,
                           int32_t *err, hipStream_t stream);

hipError_t launch_partial_attention(const dcpmla_geom &g, int groups, const void *q,
                                    const void *q_split, const float *q_inv_scale,
                                    const void *kv_pool, float kv_scale, float softmax_scale,
                                    const dcpmla_meta &m, void *workspace, void *out_rank,
                                    float *lse_rank, hipStream_t stream);

hipError_t launch_split_q(int64_t rows, const void *q, void *split, float *inv_scale, hipStream_t stream);

hipError_t launch_merge_segments(const dcpmla_geom &g, int groups, const dcpmla_meta &m,
                                 const void *workspace, void *out_rank, float *lse_rank,
                                 hipStream_t stream);

hipError_t launch_merge_ranks(int world, int64_t rows, const void *out_ranks,
                              const float *lse_ranks, void *out, float *lse, hipStream_t stream);

hipError_t launch_merge_segments_dense(int64_t rows, int nseg, const float *o_seg,
                                       const float *lse2_seg, void *out, float *lse,
                                       hipStream_t stream);

hipError_t launch_a2a_pack(int world, int64_t tokens, int heads, int dim, const void *out_rank,
                           const float *lse_rank, void *send, hipStream_t stream);

hipError_t launch_a2a_combine(int world, int64_t tokens, int heads_local, int dim, const void *recv,
                              void *out, float *lse, hipStream_t stream);

hipError_t launch_project_heads(int64_t tokens, int heads, int dv, const void *o, const void *wvt,
                                void *out, hipStream_t stream);

}  // namespace dcpmla
