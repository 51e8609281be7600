/*
 * dcpmla.h -- C ABI of the decode-context-parallel (DCP) MLA causal-verification
 * library for AMD Instinct MI355X (gfx950).
 *
 * The problem, as the pages state it.  Under DCP the latent KV cache of an MLA
 * model is sharded along the sequence: with DCP world W and interleave S,
 * global token p lives on rank (p // S) % W ("Context Parallel Guide (PCP &
 * DCP)", --dcp-config table, interleave_size).  Block tables hold *virtual*
 * block ids shared by every rank; on each rank one id names that rank's own
 * physical block of block_size consecutive rank-local tokens (same page, "How
 * it works" item 1).  Every rank receives all gathered query heads, runs
 * attention over its local tokens and returns a partial output with its
 * log-sum-exp; the partials are then LSE-combined (same page, "How it works"
 * item 3).  For causal multi-token verification each verify row i of a
 * sequence with ctx cached tokens (the qlen verify tokens included) sees the
 * global positions [0, ctx - qlen + 1 + i); its rank-local window is the
 * owned subset, always a prefix of the rank-local token list
 * ("[ROCm][MLA][DCP] Support causal multi-token verification", vLLM PR
 * #51705, "Implementation" items 1-3).
 *
 * Fixed dimensions: query/key width 576 (512 latent + 64 rope), value width
 * 512 (the first 512 dims of the same cached latent vector).
 *
 * Conventions for every call:
 *  - Pointers named as device pointers must be device memory of the current
 *    HIP device; the caller owns all buffers.  Host-only calls touch no GPU.
 *  - Every launch is asynchronous on `stream`; nothing synchronises.
 *  - Invalid arguments are refused before any launch with a negative status.
 *  - Data-dependent violations found on the device (see DCPMLA_ERR_*) never
 *    read or write out of bounds: the affected row is clamped and a bit is
 *    OR-ed into the caller's device error word, which the caller reads after
 *    synchronising.
 *  - Output buffers must not overlap any input buffer (DCPMLA_E_ALIAS).
 *  - Launch shapes depend only on the geometry, never on device data, so a
 *    call sequence can be captured in a HIP graph once and replayed.
 */
#ifndef DCPMLA_H
#define DCPMLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCPMLA_D_QK 576
#define DCPMLA_D_V 512

/* Status codes returned by every call (0 = success). */
typedef enum {
  DCPMLA_OK = 0,
  DCPMLA_E_INVALID = -1,     /* bad geometry, null pointer or out-of-range scalar */
  DCPMLA_E_ALIAS = -2,       /* an output buffer overlaps an input buffer */
  DCPMLA_E_WORKSPACE = -3,   /* workspace smaller than dcpmla_workspace_bytes() */
  DCPMLA_E_UNSUPPORTED = -4, /* valid request the library does not implement */
  DCPMLA_E_HIP = -5,         /* a HIP runtime call failed (launch, attribute query) */
  DCPMLA_E_SCRATCH = -6      /* request larger than the library's static scratch array */
} dcpmla_status;

/* Latent-cache element formats. */
enum {
  DCPMLA_KV_BF16 = 0,     /* bfloat16 */
  DCPMLA_KV_FP8_E4M3 = 1  /* OCP FP8 E4M3 (max 448) with one per-tensor float scale */
};

/*
 * Which global positions a row sees.  CAUSAL: verify row i of a sequence with
 * ctx cached tokens sees [0, ctx - qlen + 1 + i) ("[ROCm][MLA][DCP] Support
 * causal multi-token verification", "Implementation" item 1).  BLOCK: a
 * bidirectional draft block -- every row sees the whole cache [0, ctx)
 * ("Context Parallel Guide (PCP & DCP)", "DSpark (Kimi-K3)": the draft block
 * attends the whole block, so no mask is placed on global positions).
 */
enum {
  DCPMLA_BOUNDARY_CAUSAL = 0,
  DCPMLA_BOUNDARY_BLOCK = 1
};

/*
 * How an FP8-cache attention multiplies the BF16 query against the cache.
 * SPLIT (default): as two E4M3 terms that sum to the query exactly (see
 * dcpmla_split_q()), so the result is the BF16-query attention.  FP8: as one
 * E4M3 term per element with a per-head-row power-of-two scale -- the
 * quantised FP8 query of "Context Parallel Guide (PCP & DCP)", "How it
 * works" item 4 (decode gathers an FP8 query for an FP8 cache); the result
 * is attention with that quantised query, and the query products take half
 * the matrix work.  FP8 requires an FP8 cache.
 */
enum {
  DCPMLA_Q_SPLIT = 0,
  DCPMLA_Q_FP8 = 1
};

/*
 * How an FP8-cache attention feeds the softmax probabilities p to the p.v
 * products (the value operand is the E4M3 cache itself).  SPLIT (default): p,
 * scaled by a power of two, as an E4M3 term plus an E5M2 remainder -- about 7
 * significant bits, on a par with a BF16 p -- in two FP8 products; the output
 * is normalised by the sum of exactly the values multiplied.  FP8: the E4M3
 * term alone, one product (half the p.v matrix work; the probabilities carry
 * 4 significant bits), after "Context Parallel Guide (PCP & DCP)", "How it
 * works" item 4 and "Sparse DCP persistent attention and gqa=64" (decode runs
 * MLA with FP8 operands against an FP8 cache).  FP8 requires an FP8 cache.
 */
enum {
  DCPMLA_P_SPLIT = 0,
  DCPMLA_P_FP8 = 1
};

/* Bits of the device error word. */
enum {
  DCPMLA_ERR_CTX_LT_QLEN = 1,    /* ctx < qlen: rows whose boundary would be < 1 get no tokens */
  DCPMLA_ERR_TABLE_CAPACITY = 2, /* a row needs more blocks than max_blocks_per_seq: row clamped */
  DCPMLA_ERR_LOCAL_PAGES = 4,    /* a row needs more subpages than max_local_pages: row clamped */
  DCPMLA_ERR_BLOCK_ID = 8,       /* a used block id lies outside [0, num_blocks): row cut there */
  DCPMLA_ERR_PAGE_RANGE = 16,    /* attention met a subpage outside the pool: tokens read as 0 */
  DCPMLA_ERR_TOKEN = 32,         /* KV write: bad sequence id / position: token dropped */
  DCPMLA_ERR_KERNARG = 64        /* attention: the kernel argument block was not found at offset 0 of
                                    the kernel-argument segment (a toolchain ABI change); the
                                    launch's outputs are not valid */
};

/*
 * Geometry of one DCP group and one verification batch.  Validated by
 * dcpmla_validate() with the pages' startup rules ("Context Parallel Guide",
 * interleave_size: 1 <= S <= block_size, block_size % S == 0 when S > 1,
 * S > 1 needs W > 1).
 */
typedef struct dcpmla_geom {
  int32_t dcp_world;          /* W >= 1 */
  int32_t interleave;         /* S */
  int32_t block_size;         /* tokens per physical block on each rank */
  int32_t qlen;               /* verify rows per sequence, >= 1 */
  int32_t num_heads;          /* gathered query heads H >= 1 */
  int32_t batch;              /* sequences B >= 1 */
  int32_t max_blocks_per_seq; /* block_table row width (entries) */
  int32_t max_local_pages;    /* static per-row bound on subpages; page_table row width */
  int32_t kv_dtype;           /* DCPMLA_KV_BF16 or DCPMLA_KV_FP8_E4M3 */
  int32_t groups;             /* persistent workgroups of the attention kernel; 0 = one per
                                 compute unit of the current device */
  int64_t num_blocks;         /* physical blocks in each rank's pool */
  int32_t row_boundary;       /* DCPMLA_BOUNDARY_CAUSAL (default) or DCPMLA_BOUNDARY_BLOCK */
  int32_t q_format;           /* DCPMLA_Q_SPLIT (default) or DCPMLA_Q_FP8 (FP8 cache only) */
  int32_t p_format;           /* DCPMLA_P_SPLIT (default) or DCPMLA_P_FP8 (FP8 cache only) */
} dcpmla_geom;

/*
 * The per-rank verify view, built once per forward by dcpmla_build_metadata()
 * and reused by every attention call of that forward (PR #51705,
 * "Implementation" items 4-5: the builder owns the decision and allocates
 * stable row metadata).  Row index = b*qlen + i.  All device int32.
 */
typedef struct dcpmla_meta {
  int32_t *row_local_len;   /* [B*qlen]   rank-local tokens visible to the row */
  int32_t *page_table;      /* [B*qlen, max_local_pages] subpage ids, -1 = unused */
  int32_t *last_page_len;   /* [B*qlen]   tokens in the row's last subpage (0 if none) */
  int32_t *err;             /* [1]        device error word (DCPMLA_ERR_* bits), OR-ed */
  int32_t *work;            /* [dcpmla_work_ints()] split-KV work partition and one zero
                               latent row that stands in for tokens outside a sequence
                               (opaque; written by dcpmla_build_metadata) */
} dcpmla_meta;

/* Host only.  DCPMLA_OK or DCPMLA_E_INVALID. */
int dcpmla_validate(const dcpmla_geom *geom);

/*
 * Host only.  Subpage size the segmented kernel reads: the largest power of
 * two dividing block_size, capped at 128 (PR #51705, review thread on
 * _segmented_mla_page_size).  DCPMLA_E_INVALID for block_size < 1.
 */
int32_t dcpmla_subpage_size(int32_t block_size);

/* Host only.  Length in int32 of dcpmla_meta.work; negative status if invalid. */
int64_t dcpmla_work_ints(const dcpmla_geom *geom);

/*
 * Bytes of scratch dcpmla_partial_attention() needs (split-KV partials, then
 * the split query of an FP8-cache launch).  Host only when
 * geom->groups > 0; with groups == 0 it asks the current device for its
 * compute-unit count (DCPMLA_E_HIP without a device).  Negative on error.
 */
int64_t dcpmla_workspace_bytes(const dcpmla_geom *geom);

/*
 * Interleaved KV write for one rank ("Context Parallel Guide", "How it works"
 * item 2 and the DSpark bullet: tokens go through a slot mapping, -1 for
 * tokens the rank does not own).  For each of num_tokens tokens with
 * sequence seq_ids[t] and global position positions[t], if rank owns the
 * position, copies its 576-element latent row latents[t] (already in the
 * cache format) into the rank's pool at
 *   block_table[b][li / block_size] * block_size + li % block_size,
 * li = (p / (S*W)) * S + p % S, and stores that pool row in slot_mapping[t];
 * otherwise stores -1.  Device pointers: seq_ids, positions [T] int32;
 * latents [T, 576] cache elements; block_table [B, max_blocks_per_seq];
 * kv_pool [num_blocks, block_size, 576]; slot_mapping [T] int32; err [1].
 * Bad ids/positions or block ids set DCPMLA_ERR_TOKEN / DCPMLA_ERR_BLOCK_ID.
 */
int dcpmla_write_kv(const dcpmla_geom *geom, int32_t rank, int64_t num_tokens,
                    const int32_t *seq_ids, const int32_t *positions, const void *latents,
                    const int32_t *block_table, void *kv_pool, int32_t *slot_mapping,
                    int32_t *err, hipStream_t stream);

/*
 * Verify-view builder for one rank (PR #51705, "Implementation" items 1-2;
 * per-row length formula from "[Spec decode] Support Kimi-K3 DCP with
 * DSpark", vLLM PR #52188, review thread):
 *   g   = ctx[b] - qlen + 1 + i                     (global causal boundary)
 *   len = (g / (W*S)) * S + clamp(g % (W*S) - rank*S, 0, S)
 *   P   = dcpmla_subpage_size(block_size), ppb = block_size / P
 *   page j < ceil(len/P):  block_table[b][j / ppb] * ppb + j % ppb
 * then the split-KV work partition.  Reads block_table only below the
 * row's page count (bounded load).  ctx_lens [B], block_table [B,
 * max_blocks_per_seq] device int32; meta buffers as in dcpmla_meta.  Does not
 * clear meta->err.
 */
int dcpmla_build_metadata(const dcpmla_geom *geom, int32_t rank, const int32_t *ctx_lens,
                          const int32_t *block_table, const dcpmla_meta *meta,
                          hipStream_t stream);

/*
 * Segmented split-KV MLA attention for one rank (PR #51705, "Implementation"
 * item 3): each (sequence, head-row tile, KV range) piece produces either the
 * finished rank output or an unreduced partial with base-2 softmax
 * statistics in the workspace (partial outputs as fp16 values of o / kv_scale
 * with an FP8 cache, whose magnitude the E4M3 maximum 448 bounds, and as float
 * with a BF16 cache).  Scores are q . k * softmax_scale over all 576
 * dims; the cached elements are multiplied by kv_scale (1 for BF16 caches).
 * q [B, qlen, H, 576] bf16; kv_pool [num_blocks, block_size, 576] in
 * geom->kv_dtype; out_rank [B, qlen, H, 512] bf16 and lse_rank [B, qlen, H]
 * float (natural log) receive the rows finished here; workspace of
 * dcpmla_workspace_bytes() bytes.  With an FP8 cache the call first writes
 * dcpmla_split_q() of q into the workspace and runs q . k on the FP8 matrix
 * units as the two exact E4M3 terms.  Must be followed by
 * dcpmla_merge_segments() on the same stream.
 */
int dcpmla_partial_attention(const dcpmla_geom *geom, const void *q, const void *kv_pool,
                             float kv_scale, float softmax_scale, const dcpmla_meta *meta,
                             void *workspace, int64_t workspace_bytes, void *out_rank,
                             float *lse_rank, hipStream_t stream);

/*
 * dcpmla_partial_attention() for an FP8 cache with the query given already
 * split (dcpmla_split_q() output): q_split of dcpmla_split_q_bytes(B*qlen*H)
 * bytes and q_inv_scale [B*qlen*H] float, device memory.  For a DCP group the split is
 * done once per forward ("Context Parallel Guide", "How it works" item 4: the
 * query is gathered once per decode step; each rank may split its own head
 * slice before the gather, the split form having the size of the BF16
 * query), and every rank's call reads it.  DCPMLA_E_INVALID with a BF16
 * cache; other arguments, the workspace and the errors as in
 * dcpmla_partial_attention().
 */
int dcpmla_partial_attention_split(const dcpmla_geom *geom, const void *q_split,
                                   const float *q_inv_scale, const void *kv_pool, float kv_scale,
                                   float softmax_scale, const dcpmla_meta *meta, void *workspace,
                                   int64_t workspace_bytes, void *out_rank, float *lse_rank,
                                   hipStream_t stream);

/*
 * Segment merge (PR #51705, "Implementation" item 3 and commit message: the
 * base-2 statistics become a BF16 output plus a natural-log LSE):
 *   L2 = log2 sum_s 2^lse2_s,  O = sum_s 2^(lse2_s - L2) o_s,  LSE = L2 * ln 2
 * for every row split across workgroups; rows with no visible token get
 * O = 0 and LSE = -inf.  Arguments as in dcpmla_partial_attention().
 */
int dcpmla_merge_segments(const dcpmla_geom *geom, const dcpmla_meta *meta,
                          const void *workspace, int64_t workspace_bytes, void *out_rank,
                          float *lse_rank, hipStream_t stream);

/* dcpmla_partial_attention() followed by dcpmla_merge_segments(). */
int dcpmla_rank_attention(const dcpmla_geom *geom, const void *q, const void *kv_pool,
                          float kv_scale, float softmax_scale, const dcpmla_meta *meta,
                          void *workspace, int64_t workspace_bytes, void *out_rank,
                          float *lse_rank, hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * dcpmla_rank_attention() without the workspace argument.  The split-KV
 * partials and the split query go to a device array inside the library,
 * DCPMLA_STATIC_SCRATCH_BYTES (160 MiB) on every GPU it runs on, held until
 * the process ends; the call itself allocates nothing (no hipMalloc, hipFree
 * or allocating library routine).  The request needs
 * dcpmla_workspace_bytes(geom) bytes of it (with geom->groups = 0 that is
 * about 134 MB for the 256-CU grid plus 1,156 bytes per head-row, so up to
 * about 28,000 head-rows); a larger request returns DCPMLA_E_SCRATCH before
 * any launch (a smaller geom->groups needs less).  The array keeps the last
 * call's contents; nothing in it has to start at zero.  All calls on one GPU
 * share its array, so calls that overlap in time on one GPU (on different
 * streams, or from different threads) race and must be ordered by the
 * caller.  Other arguments, results and errors as in dcpmla_rank_attention();
 * the results are those of dcpmla_rank_attention() with the same geometry,
 * bit for bit.
 */
#define DCPMLA_STATIC_SCRATCH_BYTES (160LL << 20)
int dcpmla_rank_attention_static(const dcpmla_geom *geom, const void *q, const void *kv_pool,
                                 float kv_scale, float softmax_scale, const dcpmla_meta *meta,
                                 void *out_rank, float *lse_rank, hipStream_t stream);

/* Host only.  DCPMLA_STATIC_SCRATCH_BYTES. */
int64_t dcpmla_static_scratch_bytes(void);

/*
 * Exact two-term E4M3 split of BF16 query rows, the form in which an FP8-cache
 * dcpmla_partial_attention() multiplies q against the cache (the query is
 * BF16, PR #51705; the cache FP8 E4M3 with a per-tensor scale, "Context
 * Parallel Guide", "How it works" item 4).  Per row, k is the largest
 * integer with max|q| * 2^k <= 448, hi the E4M3 code nearest x = q * 2^k
 * (ties to even) and lo the code nearest x - hi.  BF16 has 8 significant bits
 * and E4M3 4, so q = (hi + lo) * 2^-k exactly for |x| >= 2^-2, and within
 * 2^-10 * 2^-k below.  q [rows, 576] bf16 (device); inv_scale [rows] float =
 * 2^-k; q_split dcpmla_split_q_bytes(rows) bytes holding the codes tiled for
 * the attention kernel's loads: rows in blocks of 32 (the last block padded),
 * each block 36 chunks of 1 KiB; chunk c = 4t + 2 term + half (t < 9, term 0
 * = hi, 1 = lo, half < 2) holds at bytes 16 (32 g + i) .. +15 the codes of
 * row 32 n + i of block n for dims 64t + 32g + 16 half .. +15 (g < 2).  The
 * padding rows of the last block are not written.  Outputs may not overlap
 * q or each other (DCPMLA_E_ALIAS).
 */
int dcpmla_split_q(int64_t rows, const void *q, void *q_split, float *inv_scale, hipStream_t stream);

/* Host only.  Bytes of q_split for `rows` head-rows (DCPMLA_E_INVALID if out of range). */
int64_t dcpmla_split_q_bytes(int64_t rows);

/*
 * Cross-rank LSE merge ("Context Parallel Guide", enable_project_before_merge:
 * a per-(token, head) scalar weight plus a cross-rank sum; PR #51705: an
 * empty rank has LSE = -inf and contributes nothing):
 *   LSE = ln sum_r exp(LSE_r),  O = sum_r exp(LSE_r - LSE) O_r   (BF16 out)
 * Rows empty on every rank get O = 0, LSE = -inf.  out_ranks [W, rows, 512]
 * bf16 and lse_ranks [W, rows] float, contiguous; out [rows, 512] bf16 and
 * lse [rows] float; rows = B * qlen * H.
 */
int dcpmla_merge_ranks(int32_t dcp_world, int64_t rows, const void *out_ranks,
                       const float *lse_ranks, void *out, float *lse, hipStream_t stream);

/*
 * Base-2 segment merge on a plain layout: o_seg [rows, nseg, 512] float and
 * lse2_seg [rows, nseg] float -> out [rows, 512] bf16, lse [rows] float
 * (natural log).  Same arithmetic as dcpmla_merge_segments(); for callers
 * that keep their own split-KV partials.
 */
int dcpmla_merge_segments_dense(int64_t rows, int32_t nseg, const float *o_seg,
                                const float *lse2_seg, void *out, float *lse,
                                hipStream_t stream);

/*
 * The exchange around the cross-rank merge ("Context Parallel Guide (PCP &
 * DCP)", comm_backend a2a): each rank sends every peer that peer's slice of
 * heads of its partial, with the fp32 LSE packed alongside as two 16-bit
 * halves of the bf16 message (an exact round trip), and the combine is done
 * locally.  A message row is dim bf16 values, then the LSE's low and high 16
 * bits, then six zeros: dcpmla_a2a_message_elems(dim) = dim + 8 elements
 * (16-byte aligned).  The all-to-all itself is a collective outside this
 * library: block p of rank r's send buffer becomes block r of rank p's receive
 * buffer.
 */
int64_t dcpmla_a2a_message_elems(int32_t dim);

/*
 * Pack one rank's partial: out_rank [tokens, heads, dim] bf16 and lse_rank
 * [tokens, heads] float (natural log) -> send [W][tokens][heads/W][dim + 8]
 * bf16, block p holding heads [p*heads/W, (p+1)*heads/W).  heads % W == 0,
 * dim a multiple of 8 in [8, 512] (512 = latent output, smaller = projected
 * by dcpmla_project_heads).  DCPMLA_E_ALIAS if send overlaps an input.
 */
int dcpmla_a2a_pack(int32_t dcp_world, int64_t tokens, int32_t heads, int32_t dim, const void *out_rank,
                    const float *lse_rank, void *send, hipStream_t stream);

/*
 * Local combine after the exchange: recv [W][tokens][heads_local][dim + 8]
 * (block r from rank r) -> out [tokens, heads_local, dim] bf16 and lse
 * [tokens, heads_local] float: L = ln sum_r e^LSE_r, O = sum_r e^(LSE_r - L) O_r,
 * ranks with LSE = -inf weigh nothing; rows with no mass anywhere get O = 0,
 * LSE = -inf.  Same arithmetic, in the same order, as dcpmla_merge_ranks().
 */
int dcpmla_a2a_combine(int32_t dcp_world, int64_t tokens, int32_t heads_local, int32_t dim,
                       const void *recv, void *out, float *lse, hipStream_t stream);

/*
 * Project before merge ("Context Parallel Guide (PCP & DCP)",
 * enable_project_before_merge): W_V is a per-head linear map and the merge is
 * a per-(token, head) scalar weighting plus a cross-rank sum, so W_V can be
 * applied to each rank's partial first and the exchange carries v_head_dim
 * values per head instead of 512.  out [tokens, heads, v_head_dim] bf16 =
 * o [tokens, heads, 512] bf16 times W_V[h] [512, v_head_dim], with W_V given
 * transposed as w_v_t [heads, v_head_dim, 512] bf16; fp32 accumulation.
 * v_head_dim a multiple of 32 up to 512.
 */
int dcpmla_project_heads(int64_t tokens, int32_t heads, int32_t v_head_dim, const void *o,
                         const void *w_v_t, void *out, hipStream_t stream);

/* Static description of a status code. */
const char *dcpmla_strerror(int status);

/*
 * Device description used to state roofline peaks next to measurements (the
 * measurement of the segmented kernel is set against the binding HBM or
 * MFMA roofline; the peaks are the chip's, not the pages').  Fills *out for
 * HIP device `device`; DCPMLA_E_INVALID for a null pointer, DCPMLA_E_HIP if
 * the runtime cannot describe the device.  Host call, no kernel launch.
 */
typedef struct dcpmla_device_info {
  int32_t compute_units;      /* multiProcessorCount */
  int32_t clock_khz;          /* peak shader clock */
  int32_t memory_clock_khz;   /* memory clock as reported by the runtime */
  int32_t memory_bus_bits;    /* memory interface width */
  int64_t lds_bytes_per_block;
  char arch[64];              /* gcnArchName, NUL-terminated */
} dcpmla_device_info;
int dcpmla_get_device_info(int32_t device, dcpmla_device_info *out);

#ifdef __cplusplus
}
#endif

#endif /* DCPMLA_H */
