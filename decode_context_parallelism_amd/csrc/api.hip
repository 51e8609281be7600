// C ABI entry points: argument validation, aliasing checks, launches.
#include <string.h>

#include <cstring>

#include "common.h"
#include "launch.h"

namespace {

using namespace dcpmla;

constexpr int kMaxGroups = 1024;

struct Range {
  const void *p;
  int64_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
  return a0 < b1 && b0 < a1;
}

// every output must be disjoint from every input and from the other outputs
bool any_alias(const Range *outs, int nout, const Range *ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

int elem_bytes(const dcpmla_geom *g) { return g->kv_dtype == DCPMLA_KV_FP8_E4M3 ? 1 : 2; }

int resolve_groups(const dcpmla_geom *g, int *groups) {
  if (g->groups > 0) {
    *groups = g->groups;
    return DCPMLA_OK;
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DCPMLA_E_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return DCPMLA_E_HIP;
  if (cus < 1) return DCPMLA_E_HIP;
  *groups = cus < kMaxGroups ? cus : kMaxGroups;
  return DCPMLA_OK;
}

int meta_ok(const dcpmla_geom *g, const dcpmla_meta *m) {
  if (!m || !m->row_local_len || !m->page_table || !m->last_page_len || !m->err || !m->work)
    return 0;
  (void)g;
  return 1;
}

void meta_ranges(const dcpmla_geom *g, const dcpmla_meta *m, Range *r) {
  const int64_t rows = (int64_t)g->batch * g->qlen;
  r[0] = {m->row_local_len, rows * 4};
  r[1] = {m->page_table, rows * g->max_local_pages * 4};
  r[2] = {m->last_page_len, rows * 4};
  r[3] = {m->err, 4};
  r[4] = {m->work, work_ints(g->batch) * 4};
}

int hip_status(hipError_t e) { return e == hipSuccess ? DCPMLA_OK : DCPMLA_E_HIP; }

}  // namespace

extern "C" {

int dcpmla_validate(const dcpmla_geom *g) {
  if (!g) return DCPMLA_E_INVALID;
  if (g->dcp_world < 1 || g->block_size < 1 || g->qlen < 1 || g->num_heads < 1 || g->batch < 1)
    return DCPMLA_E_INVALID;
  // interleave rules asserted at startup by the pages' configuration
  if (g->interleave < 1 || g->interleave > g->block_size) return DCPMLA_E_INVALID;
  if (g->interleave > 1 && (g->block_size % g->interleave != 0 || g->dcp_world < 2))
    return DCPMLA_E_INVALID;
  if (g->max_blocks_per_seq < 1 || g->max_local_pages < 1 || g->num_blocks < 1)
    return DCPMLA_E_INVALID;
  if (g->kv_dtype != DCPMLA_KV_BF16 && g->kv_dtype != DCPMLA_KV_FP8_E4M3) return DCPMLA_E_INVALID;
  if (g->groups < 0 || g->groups > kMaxGroups) return DCPMLA_E_INVALID;
  if (g->q_format != DCPMLA_Q_SPLIT && g->q_format != DCPMLA_Q_FP8) return DCPMLA_E_INVALID;
  if (g->q_format == DCPMLA_Q_FP8 && g->kv_dtype != DCPMLA_KV_FP8_E4M3) return DCPMLA_E_INVALID;
  if (g->p_format != DCPMLA_P_SPLIT && g->p_format != DCPMLA_P_FP8) return DCPMLA_E_INVALID;
  if (g->p_format == DCPMLA_P_FP8 && g->kv_dtype != DCPMLA_KV_FP8_E4M3) return DCPMLA_E_INVALID;
  if (g->row_boundary != DCPMLA_BOUNDARY_CAUSAL && g->row_boundary != DCPMLA_BOUNDARY_BLOCK)
    return DCPMLA_E_INVALID;
  // index arithmetic stays in 32 bits on the device
  const int P = subpage_size(g->block_size);
  const int64_t pages = g->num_blocks * (g->block_size / P);
  if (g->num_blocks * (int64_t)g->block_size >= ((int64_t)1 << 31)) return DCPMLA_E_INVALID;
  if (pages >= ((int64_t)1 << 31)) return DCPMLA_E_INVALID;
  const int64_t max_tokens = (int64_t)g->max_local_pages * P;
  if (max_tokens >= ((int64_t)1 << 31)) return DCPMLA_E_INVALID;
  const int64_t units = (int64_t)g->batch * n_mtiles(g->qlen, g->num_heads) *
                        ((max_tokens + kStageTokens - 1) / kStageTokens);
  if (units >= ((int64_t)1 << 31)) return DCPMLA_E_INVALID;
  if ((int64_t)g->batch * g->qlen * g->num_heads >= ((int64_t)1 << 31) / kDqk) return DCPMLA_E_INVALID;
  if ((int64_t)g->batch * g->max_blocks_per_seq >= ((int64_t)1 << 31)) return DCPMLA_E_INVALID;
  return DCPMLA_OK;
}

int32_t dcpmla_subpage_size(int32_t block_size) {
  if (block_size < 1) return DCPMLA_E_INVALID;
  return subpage_size(block_size);
}

int64_t dcpmla_work_ints(const dcpmla_geom *g) {
  const int v = dcpmla_validate(g);
  if (v != DCPMLA_OK) return v;
  return work_ints(g->batch);
}

int64_t dcpmla_workspace_bytes(const dcpmla_geom *g) {
  const int v = dcpmla_validate(g);
  if (v != DCPMLA_OK) return v;
  int groups = 0;
  const int r = resolve_groups(g, &groups);
  if (r != DCPMLA_OK) return r;
  return ws_total_bytes(groups, (int64_t)g->batch * g->qlen * g->num_heads);
}

int dcpmla_write_kv(const dcpmla_geom *g, int32_t rank, int64_t num_tokens, const int32_t *seq_ids,
                    const int32_t *positions, const void *latents, const int32_t *block_table,
                    void *kv_pool, int32_t *slot_mapping, int32_t *err, hipStream_t stream) {
  const int v = dcpmla_validate(g);
  if (v != DCPMLA_OK) return v;
  if (rank < 0 || rank >= g->dcp_world || num_tokens < 0) return DCPMLA_E_INVALID;
  if (num_tokens > 0 && (!seq_ids || !positions || !latents || !slot_mapping))
    return DCPMLA_E_INVALID;
  if (!block_table || !kv_pool || !err) return DCPMLA_E_INVALID;
  const int64_t row_bytes = (int64_t)kDqk * elem_bytes(g);
  const Range ins[] = {{seq_ids, num_tokens * 4}, {positions, num_tokens * 4},
                       {latents, num_tokens * row_bytes},
                       {block_table, (int64_t)g->batch * g->max_blocks_per_seq * 4}};
  const Range outs[] = {{kv_pool, g->num_blocks * g->block_size * row_bytes},
                        {slot_mapping, num_tokens * 4},
                        {err, 4}};
  if (any_alias(outs, 3, ins, 4)) return DCPMLA_E_ALIAS;
  return hip_status(launch_write_kv(*g, rank, num_tokens, seq_ids, positions, latents, block_table,
                                    kv_pool, slot_mapping, err, stream));
}

int dcpmla_build_metadata(const dcpmla_geom *g, int32_t rank, const int32_t *ctx_lens,
                          const int32_t *block_table, const dcpmla_meta *m, hipStream_t stream) {
  const int v = dcpmla_validate(g);
  if (v != DCPMLA_OK) return v;
  if (rank < 0 || rank >= g->dcp_world || !ctx_lens || !block_table || !meta_ok(g, m))
    return DCPMLA_E_INVALID;
  Range outs[5];
  meta_ranges(g, m, outs);
  const Range ins[] = {{ctx_lens, (int64_t)g->batch * 4},
                       {block_table, (int64_t)g->batch * g->max_blocks_per_seq * 4}};
  if (any_alias(outs, 5, ins, 2)) return DCPMLA_E_ALIAS;
  return hip_status(launch_build_metadata(*g, rank, ctx_lens, block_table, *m, stream));
}

// q_in: the query operand's buffers (the BF16 query, or the split query and
// its scales)
static int attention_checks(const dcpmla_geom *g, const Range *q_in, int n_q, const void *kv_pool,
                            const dcpmla_meta *m, const void *workspace, int64_t workspace_bytes,
                            const void *out_rank, const float *lse_rank, int *groups) {
  const int v = dcpmla_validate(g);
  if (v != DCPMLA_OK) return v;
  if (!meta_ok(g, m) || !workspace || !out_rank || !lse_rank) return DCPMLA_E_INVALID;
  const int r = resolve_groups(g, groups);
  if (r != DCPMLA_OK) return r;
  const int64_t rows = (int64_t)g->batch * g->qlen * g->num_heads;
  if (workspace_bytes < ws_total_bytes(*groups, rows)) return DCPMLA_E_WORKSPACE;
  Range mr[5];
  meta_ranges(g, m, mr);
  Range ins[7] = {{kv_pool, g->num_blocks * g->block_size * (int64_t)kDqk * elem_bytes(g)},
                 mr[0], mr[1], mr[2], mr[4]};
  int n_in = 5;
  for (int i = 0; i < n_q; ++i) ins[n_in++] = q_in[i];
  const Range outs[] = {{workspace, workspace_bytes}, {out_rank, rows * kDv * 2}, {lse_rank, rows * 4}};
  if (any_alias(outs, 3, ins, n_in)) return DCPMLA_E_ALIAS;
  // the error word is written too; it may not share memory with anything else
  const Range err_out[] = {mr[3]};
  if (any_alias(err_out, 1, outs, 3) || any_alias(err_out, 1, ins, n_in)) return DCPMLA_E_ALIAS;
  return DCPMLA_OK;
}

static bool scales_ok(float kv_scale, float softmax_scale) {
  return kv_scale > 0.f && softmax_scale > 0.f && kv_scale != __builtin_huge_valf() &&
         softmax_scale != __builtin_huge_valf();
}

int dcpmla_partial_attention(const dcpmla_geom *g, const void *q, const void *kv_pool,
                             float kv_scale, float softmax_scale, const dcpmla_meta *m,
                             void *workspace, int64_t workspace_bytes, void *out_rank,
                             float *lse_rank, hipStream_t stream) {
  if (!q || !kv_pool || !g) return DCPMLA_E_INVALID;
  if (!scales_ok(kv_scale, softmax_scale)) return DCPMLA_E_INVALID;
  int groups = 0;
  const Range qr[] = {{q, (int64_t)g->batch * g->qlen * g->num_heads * kDqk * 2}};
  const int c = attention_checks(g, qr, 1, kv_pool, m, workspace, workspace_bytes, out_rank, lse_rank,
                                 &groups);
  if (c != DCPMLA_OK) return c;
  return hip_status(launch_partial_attention(*g, groups, q, nullptr, nullptr, kv_pool, kv_scale,
                                             softmax_scale, *m, workspace, out_rank, lse_rank, stream));
}

int dcpmla_partial_attention_split(const dcpmla_geom *g, const void *q_split, const float *q_inv_scale,
                                   const void *kv_pool, float kv_scale, float softmax_scale,
                                   const dcpmla_meta *m, void *workspace, int64_t workspace_bytes,
                                   void *out_rank, float *lse_rank, hipStream_t stream) {
  if (!q_split || !q_inv_scale || !kv_pool || !g) return DCPMLA_E_INVALID;
  if (g->kv_dtype != DCPMLA_KV_FP8_E4M3) return DCPMLA_E_INVALID;
  if (!scales_ok(kv_scale, softmax_scale)) return DCPMLA_E_INVALID;
  int groups = 0;
  const int64_t rows = (int64_t)g->batch * g->qlen * g->num_heads;
  const Range qr[] = {{q_split, qsplit_bytes(rows)}, {q_inv_scale, rows * 4}};
  const int c = attention_checks(g, qr, 2, kv_pool, m, workspace, workspace_bytes, out_rank, lse_rank,
                                 &groups);
  if (c != DCPMLA_OK) return c;
  return hip_status(launch_partial_attention(*g, groups, nullptr, q_split, q_inv_scale, kv_pool, kv_scale,
                                             softmax_scale, *m, workspace, out_rank, lse_rank, stream));
}

int dcpmla_merge_segments(const dcpmla_geom *g, const dcpmla_meta *m, const void *workspace,
                          int64_t workspace_bytes, void *out_rank, float *lse_rank,
                          hipStream_t stream) {
  const int v = dcpmla_validate(g);
  if (v != DCPMLA_OK) return v;
  if (!meta_ok(g, m) || !workspace || !out_rank || !lse_rank) return DCPMLA_E_INVALID;
  int groups = 0;
  const int r = resolve_groups(g, &groups);
  if (r != DCPMLA_OK) return r;
  if (workspace_bytes < ws_bytes(groups)) return DCPMLA_E_WORKSPACE;
  const int64_t rows = (int64_t)g->batch * g->qlen * g->num_heads;
  Range mr[5];
  meta_ranges(g, m, mr);
  const Range ins[] = {{workspace, workspace_bytes}, mr[4]};
  const Range outs[] = {{out_rank, rows * kDv * 2}, {lse_rank, rows * 4}};
  if (any_alias(outs, 2, ins, 2)) return DCPMLA_E_ALIAS;
  return hip_status(launch_merge_segments(*g, groups, *m, workspace, out_rank, lse_rank, stream));
}

int dcpmla_rank_attention(const dcpmla_geom *g, const void *q, const void *kv_pool, float kv_scale,
                          float softmax_scale, const dcpmla_meta *m, void *workspace,
                          int64_t workspace_bytes, void *out_rank, float *lse_rank,
                          hipStream_t stream) {
  const int a = dcpmla_partial_attention(g, q, kv_pool, kv_scale, softmax_scale, m, workspace,
                                         workspace_bytes, out_rank, lse_rank, stream);
  if (a != DCPMLA_OK) return a;
  return dcpmla_merge_segments(g, m, workspace, workspace_bytes, out_rank, lse_rank, stream);
}

int dcpmla_merge_ranks(int32_t dcp_world, int64_t rows, const void *out_ranks,
                       const float *lse_ranks, void *out, float *lse, hipStream_t stream) {
  if (dcp_world < 1 || rows < 0) return DCPMLA_E_INVALID;
  if (rows > 0 && (!out_ranks || !lse_ranks || !out || !lse)) return DCPMLA_E_INVALID;
  if (rows * kDv >= ((int64_t)1 << 40)) return DCPMLA_E_INVALID;
  const Range ins[] = {{out_ranks, (int64_t)dcp_world * rows * kDv * 2},
                       {lse_ranks, (int64_t)dcp_world * rows * 4}};
  const Range outs[] = {{out, rows * kDv * 2}, {lse, rows * 4}};
  if (any_alias(outs, 2, ins, 2)) return DCPMLA_E_ALIAS;
  return hip_status(launch_merge_ranks(dcp_world, rows, out_ranks, lse_ranks, out, lse, stream));
}

int dcpmla_merge_segments_dense(int64_t rows, int32_t nseg, const float *o_seg,
                                const float *lse2_seg, void *out, float *lse, hipStream_t stream) {
  if (nseg < 1 || rows < 0) return DCPMLA_E_INVALID;
  if (rows > 0 && (!o_seg || !lse2_seg || !out || !lse)) return DCPMLA_E_INVALID;
  if (rows * nseg * kDv >= ((int64_t)1 << 40)) return DCPMLA_E_INVALID;
  const Range ins[] = {{o_seg, rows * nseg * kDv * 4}, {lse2_seg, rows * nseg * 4}};
  const Range outs[] = {{out, rows * kDv * 2}, {lse, rows * 4}};
  if (any_alias(outs, 2, ins, 2)) return DCPMLA_E_ALIAS;
  return hip_status(launch_merge_segments_dense(rows, nseg, o_seg, lse2_seg, out, lse, stream));
}

int64_t dcpmla_a2a_message_elems(int32_t dim) {
  if (dim < 8 || dim > kDv || dim % 8 != 0) return DCPMLA_E_INVALID;
  return (int64_t)dim + 8;
}

int64_t dcpmla_split_q_bytes(int64_t rows) {
  if (rows < 0 || rows >= ((int64_t)1 << 40) / kQSplitRow) return DCPMLA_E_INVALID;
  return qsplit_bytes(rows);
}

int dcpmla_split_q(int64_t rows, const void *q, void *q_split, float *inv_scale, hipStream_t stream) {
  if (rows < 0 || rows >= ((int64_t)1 << 40) / kQSplitRow) return DCPMLA_E_INVALID;
  if (rows > 0 && (!q || !q_split || !inv_scale)) return DCPMLA_E_INVALID;
  const Range ins[] = {{q, rows * kDqk * 2}};
  const Range outs[] = {{q_split, qsplit_bytes(rows)}, {inv_scale, rows * 4}};
  if (any_alias(outs, 2, ins, 1) || any_alias(outs, 1, outs + 1, 1)) return DCPMLA_E_ALIAS;
  return hip_status(launch_split_q(rows, q, q_split, inv_scale, stream));
}

int dcpmla_a2a_pack(int32_t dcp_world, int64_t tokens, int32_t heads, int32_t dim, const void *out_rank,
                    const float *lse_rank, void *send, hipStream_t stream) {
  if (dcp_world < 1 || tokens < 0 || heads < 1 || heads % dcp_world != 0) return DCPMLA_E_INVALID;
  if (dim < 8 || dim > kDv || dim % 8 != 0) return DCPMLA_E_INVALID;
  if (tokens > 0 && (!out_rank || !lse_rank || !send)) return DCPMLA_E_INVALID;
  const int64_t rows = tokens * heads;
  if (rows * (dim + 8) >= ((int64_t)1 << 40)) return DCPMLA_E_INVALID;
  const Range ins[] = {{out_rank, rows * dim * 2}, {lse_rank, rows * 4}};
  const Range outs[] = {{send, rows * (dim + 8) * 2}};
  if (any_alias(outs, 1, ins, 2)) return DCPMLA_E_ALIAS;
  return hip_status(launch_a2a_pack(dcp_world, tokens, heads, dim, out_rank, lse_rank, send, stream));
}

int dcpmla_a2a_combine(int32_t dcp_world, int64_t tokens, int32_t heads_local, int32_t dim,
                       const void *recv, void *out, float *lse, hipStream_t stream) {
  if (dcp_world < 1 || tokens < 0 || heads_local < 1) return DCPMLA_E_INVALID;
  if (dim < 8 || dim > kDv || dim % 8 != 0) return DCPMLA_E_INVALID;
  if (tokens > 0 && (!recv || !out || !lse)) return DCPMLA_E_INVALID;
  const int64_t rows = tokens * heads_local;
  if ((int64_t)dcp_world * rows * (dim + 8) >= ((int64_t)1 << 40)) return DCPMLA_E_INVALID;
  const Range ins[] = {{recv, (int64_t)dcp_world * rows * (dim + 8) * 2}};
  const Range outs[] = {{out, rows * dim * 2}, {lse, rows * 4}};
  if (any_alias(outs, 2, ins, 1)) return DCPMLA_E_ALIAS;
  return hip_status(launch_a2a_combine(dcp_world, tokens, heads_local, dim, recv, out, lse, stream));
}

int dcpmla_project_heads(int64_t tokens, int32_t heads, int32_t v_head_dim, const void *o,
                         const void *w_v_t, void *out, hipStream_t stream) {
  if (tokens < 0 || heads < 1 || v_head_dim < 32 || v_head_dim % 32 != 0 || v_head_dim > kDv)
    return DCPMLA_E_INVALID;
  if (tokens > 0 && (!o || !w_v_t || !out)) return DCPMLA_E_INVALID;
  if (tokens * heads * kDv >= ((int64_t)1 << 40)) return DCPMLA_E_INVALID;
  if (heads > 65535) return DCPMLA_E_INVALID;
  const Range ins[] = {{o, tokens * heads * kDv * 2}, {w_v_t, (int64_t)heads * v_head_dim * kDv * 2}};
  const Range outs[] = {{out, tokens * heads * v_head_dim * 2}};
  if (any_alias(outs, 1, ins, 2)) return DCPMLA_E_ALIAS;
  return hip_status(launch_project_heads(tokens, heads, v_head_dim, o, w_v_t, out, stream));
}

const char *dcpmla_strerror(int status) {
  switch (status) {
    case DCPMLA_OK: return "success";
    case DCPMLA_E_INVALID: return "invalid argument or geometry";
    case DCPMLA_E_ALIAS: return "an output buffer overlaps an input buffer";
    case DCPMLA_E_WORKSPACE: return "workspace too small";
    case DCPMLA_E_UNSUPPORTED: return "unsupported request";
    case DCPMLA_E_HIP: return "HIP runtime error";
    case DCPMLA_E_SCRATCH: return "request needs more than the library's static scratch array";
    default: return "unknown status";
  }
}


int dcpmla_get_device_info(int32_t device, dcpmla_device_info *out) {
  if (!out) return DCPMLA_E_INVALID;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, device) != hipSuccess) return DCPMLA_E_HIP;
  out->compute_units = p.multiProcessorCount;
  out->clock_khz = p.clockRate;
  out->memory_clock_khz = p.memoryClockRate;
  out->memory_bus_bits = p.memoryBusWidth;
  out->lds_bytes_per_block = (int64_t)p.sharedMemPerBlock;
  std::memset(out->arch, 0, sizeof(out->arch));
  std::strncpy(out->arch, p.gcnArchName, sizeof(out->arch) - 1);
  return DCPMLA_OK;
}

}  // extern "C"
