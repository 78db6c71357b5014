/*
 * step5.h -- C ABI of the Step-5 sparse-indexer (DSA/CSA) hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The path, as the TensorFold page (pull request #903, "Step-5-Preview on one
 * 256 GB Mac", commit note that turns on StepFun's CSA indexer) states it:
 *   1. the indexer keys of every completed 8-token region are summarised into
 *      an e4m3 cache: per dim, a softmax over the region's z weights the
 *      prepared k (LayerNorm with bias, NEOX rotation of dims 0..31), and the
 *      weighted mean is rounded through bf16 to e4m3;
 *   2. each query row scores every completed region before its own:
 *      sum over the KV group's heads of relu(e4m3(q_h) . summary) * w_h, with
 *      q_h the RMSNorm (scale 1 + w) and NEOX-rotated indexer query;
 *   3. the top 512 regions per KV group are kept, ordered by (-score, id);
 *   4. attention runs over those regions' tokens plus the row's own region.
 * With 512 or fewer candidates every region is selected, which is the dense
 * causal attention the indexer replaces (same page).
 *
 * Geometry rules follow vLLM's Step-5 model page ("vllm.models.step5.nvidia.
 * model", _validate_step5_dsa_parallel_geometry): indexer groups equal the
 * attention KV heads, indexer heads divide into the groups, and a KV head
 * serves 4, 8 or 16 query heads.
 *
 * Conventions for every call:
 *  - Every pointer argument is device memory owned by the caller (for
 *    example a torch tensor's data_ptr()). The library allocates nothing,
 *    frees nothing, keeps no pointer after return and holds no global state:
 *    calls on different streams are independent.
 *  - Work is enqueued on `stream` and runs asynchronously; no call
 *    synchronises. Buffers must stay alive until the stream has run the work.
 *  - Inputs are read only. Outputs named below are fully overwritten
 *    (padding included); a workspace's contents on entry do not matter and
 *    are undefined on return.
 *  - A call returns a status (never throws). Every condition checkable on
 *    the host is checked before anything is enqueued; on any error nothing is
 *    enqueued and nothing is written.
 *  - Element strides are in elements of the tensor's own type; byte strides
 *    say so.
 *  - bf16 is IEEE bfloat16, e4m3 is OCP FP8 E4M3 (e4m3fn), both raw bits.
 *  - Positions are 0-based absolute token positions. Region j holds the
 *    tokens 8j .. 8j+7. A row at position p scores the completed regions
 *    before its own, j < floor(p / 8), and always attends to its own region's
 *    tokens 8*floor(p/8) .. p.
 *  - Values that live on the device (row positions, sequence indices, region
 *    ids) cannot be checked before launch; the kernels never read or write
 *    outside the ranges the host arguments describe: a row whose position or
 *    sequence is out of range gets ids -1 and a zero output, and a region id
 *    outside 0 .. floor(p/8)-1 is skipped.
 */
#ifndef STEP5_H
#define STEP5_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer geometry. Supported: the indexer part {16, 4, 64, 32, 8, 512} with
 * 4 KV heads, q_heads 16, 32 or 64 (4, 8 or 16 per KV head) and head_dim 128
 * or 192 ({..., 16, 4, 128} is the configuration of the workloads; 64 heads
 * of 192 dims is the TensorFold page's shape of Step-5's layers). Only
 * step5_sparse_attn depends on q_heads and head_dim. Geometry that breaks
 * the rules above is STEP5_E_INVALID; other valid geometry is
 * STEP5_E_UNSUPPORTED. */
typedef struct step5_geom {
  int32_t idx_heads; /* indexer query heads (16) */
  int32_t groups;    /* indexer groups == attention KV heads (4) */
  int32_t idx_dim;   /* indexer head dim (64) */
  int32_t rope_dim;  /* NEOX-rotated leading dims of the indexer q and k (32) */
  int32_t region;    /* tokens per region (8) */
  int32_t topk;      /* regions kept per (row, group) (512) */
  int32_t q_heads;   /* attention query heads (16, 32 or 64) */
  int32_t kv_heads;  /* attention KV heads (4) */
  int32_t head_dim;  /* attention head dim (128 or 192) */
} step5_geom;

enum {
  STEP5_OK = 0,
  STEP5_E_INVALID = 1,     /* an argument is wrong: null, misaligned, negative, inconsistent */
  STEP5_E_UNSUPPORTED = 2, /* valid, but outside what this build implements */
  STEP5_E_WORKSPACE = 3,   /* workspace missing, misaligned or smaller than asked for */
  STEP5_E_HIP = 4          /* the HIP runtime refused a launch */
};

/* Flag of step5_index_score_topk: q is already the prepared e4m3 indexer
 * query [rows, idx_heads, idx_dim]; step a1 (norm, rotation, rounding) is
 * skipped and q_norm_w, q_eps, rope_cs, rope_rows are ignored. */
#define STEP5_Q_E4M3 1u

/* Flag of step5_index_append: no two rows of the call share a sequence. */
#define STEP5_APPEND_ONE_PER_SEQ 1u

/* Human-readable name of a status code (static string). */
const char* step5_status_str(int status);

/*
 * Summarise completed regions into the e4m3 summary cache.
 * [TensorFold #903, indexer commit note: k prep, region summary]
 *
 * k, z        bf16 [B, T, groups, idx_dim]: the raw indexer k and z of
 *             positions t0 .. t0+T-1 of each of B sequences. Element strides:
 *             kz_stride_b between sequences, kz_stride_t between tokens; the
 *             groups*idx_dim values of a token are contiguous. 16-byte aligned
 *             base, strides multiples of 8.
 * t0          absolute position of the first token; a multiple of region.
 * ln_w, ln_b  fp32 [idx_dim]: LayerNorm weight and bias of the indexer k
 *             (shared by the groups); ln_eps > 0 its epsilon.
 * rope_cs     bf16 [rope_rows, rope_dim]: per position, cos of the
 *             rope_dim/2 NEOX frequencies followed by their sin.
 *             rope_rows >= t0 + T.
 * summary     e4m3 [B, R_cap, groups, idx_dim], byte stride s_stride_b
 *             between sequences (a multiple of 16, >= R_cap*groups*idx_dim).
 *             Written: regions t0/region .. (t0+T)/region - 1 of every
 *             sequence (every region completed inside the span; a trailing
 *             partial region is not written). Nothing else is touched.
 *             Requires (t0 + T)/region <= R_cap.
 * B == 0 or T < region is a successful no-op.
 */
int step5_index_summarize(const step5_geom* geom, const void* k, const void* z, int64_t B,
                          int64_t T, int64_t t0, int64_t kz_stride_b, int64_t kz_stride_t,
                          const float* ln_w, const float* ln_b, float ln_eps,
                          const void* rope_cs, int64_t rope_rows, void* summary,
                          int64_t s_stride_b, int64_t R_cap, hipStream_t stream);

/*
 * Append one new token per row to the indexer's k/z rings and summarise the
 * regions those tokens complete: the cache-side work of a decode step (or of
 * a prompt chunk, one row per token).
 * [TensorFold #903: prompt-path commit note (the indexer's k and z live in
 * rings that hold one prompt chunk more than a chunk); indexer commit note
 * (every completed region is summarised, as step5_index_summarize does)]
 *
 * k_new, z_new  bf16 [rows, groups, idx_dim]: the raw indexer k and z of each
 *             row's new token; element stride new_stride_row between rows
 *             (>= groups*idx_dim, a multiple of 8); 16-byte aligned.
 * row_seq     int32 [rows] (device): the row's sequence, 0 .. B-1.
 * row_pos     int64 [rows] (device): the absolute position of its token.
 * k_ring, z_ring  bf16 [B, ring_slots, groups, idx_dim]: per sequence, the
 *             token at position p lives in slot p mod ring_slots. Element
 *             stride ring_stride_b between sequences (a multiple of 8,
 *             >= ring_slots*groups*idx_dim when B > 1); 16-byte aligned.
 *             ring_slots: a multiple of region, >= region.
 * ln_w, ln_b, ln_eps, rope_cs, rope_rows  as for step5_index_summarize.
 * summary, s_stride_b, R_cap  as for step5_index_summarize.
 *
 * Step 1: every valid row's k and z are written to ring slot
 * row_pos mod ring_slots of sequence row_seq. Step 2 (after all of step 1):
 * every valid row whose token ends a region (row_pos mod region == region-1)
 * has that region, row_pos / region, summarised from the ring slots of its
 * tokens: the same bits step5_index_summarize writes from contiguous k and
 * z. Nothing else is written. A row is valid if 0 <= row_seq < B,
 * 0 <= row_pos < rope_rows and row_pos / region < R_cap; other rows are
 * skipped.
 * Preconditions (device values, not checked): the rows of one call have
 * distinct (sequence, position) pairs, and every region completed in the
 * call has its other tokens in the ring, from this call or earlier ones:
 * the positions a call brings for one sequence span at most
 * ring_slots - region + 1 tokens (a ring one prompt chunk plus one region
 * long takes chunks of that many).
 * flags       0, or STEP5_APPEND_ONE_PER_SEQ: the caller guarantees that no
 *             two rows of the call share a sequence (a decode step); the
 *             call then runs as one launch, reading a completed region's
 *             earlier tokens from the ring and the row's own from k_new/z_new.
 *             Other bits are STEP5_E_INVALID.
 * rows == 0 is a successful no-op.
 */
int step5_index_append(const step5_geom* geom, uint32_t flags, const void* k_new,
                       const void* z_new, int64_t new_stride_row, const int32_t* row_seq, const int64_t* row_pos,
                       int32_t rows, void* k_ring, void* z_ring, int64_t B, int64_t ring_slots,
                       int64_t ring_stride_b, const float* ln_w, const float* ln_b, float ln_eps,
                       const void* rope_cs, int64_t rope_rows, void* summary, int64_t s_stride_b,
                       int64_t R_cap, hipStream_t stream);

/*
 * Score every candidate region of each row and keep the best topk per group.
 * [TensorFold #903, indexer commit note: q prep, scores, top 512 by
 * (-score, id)]
 *
 * q           without STEP5_Q_E4M3: bf16 [rows, idx_heads, idx_dim], the raw
 *             indexer query; row stride q_stride_row elements (a multiple of
 *             8). With STEP5_Q_E4M3: e4m3 [rows, idx_heads, idx_dim], row
 *             stride q_stride_row bytes (a multiple of 16).
 * q_norm_w    fp32 [idx_dim]: the RMSNorm weight w, applied as (1 + w);
 *             q_eps > 0 its epsilon.
 * rope_cs     as in step5_index_summarize. A row at p >= rope_rows cannot be
 *             prepared and counts as out of range (ids -1).
 * w_head      fp32 [idx_heads] per row: head weights w_h; w_stride_row is 0
 *             (one vector for all rows) or >= idx_heads elements.
 * row_seq     device int32 [rows]: the row's sequence (0 .. B-1).
 * row_pos     device int64 [rows]: the row's absolute position p.
 * summary     e4m3 [B, R_cap, groups, idx_dim], byte stride s_stride_b; regions
 *             j < floor(p/8) of the row's sequence must hold summaries.
 *             floor(p/8) <= R_cap. R_cap <= 524288.
 * sel_ids     out: int32 [rows, groups, topk]: for each (row, group) the ids of
 *             the min(topk, floor(p/8)) best regions in (-score, id) order
 *             (best first; equal scores by smaller id), then -1.
 * sel_scores  out, nullable: fp32 [rows, groups, topk]: their scores, 0 after
 *             the last id.
 * workspace   device scratch of at least step5_index_score_topk_workspace()
 *             bytes, 256-byte aligned.
 * rows == 0 is a successful no-op.
 */
int step5_index_score_topk(const step5_geom* geom, uint32_t flags, const void* q,
                           int64_t q_stride_row, const float* q_norm_w, float q_eps,
                           const void* rope_cs, int64_t rope_rows, const float* w_head,
                           int64_t w_stride_row, const int32_t* row_seq, const int64_t* row_pos,
                           int32_t rows, const void* summary, int64_t B, int64_t R_cap,
                           int64_t s_stride_b, int32_t* sel_ids, float* sel_scores,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes step5_index_score_topk needs for these sizes (0 if the
 * geometry or sizes are not accepted). */
size_t step5_index_score_topk_workspace(const step5_geom* geom, int32_t rows, int64_t R_cap);

/* The append half of step5_index_append_score_topk: the arguments of
 * step5_index_append that step5_index_score_topk does not have. */
typedef struct step5_append_in {
  const void* k_new;       /* bf16 [rows, groups, idx_dim], row stride new_stride_row */
  const void* z_new;
  int64_t new_stride_row;
  void* k_ring;            /* bf16 [B, ring_slots, groups, idx_dim] */
  void* z_ring;
  int64_t ring_slots;
  int64_t ring_stride_b;
  const float* ln_w;       /* the indexer k LayerNorm, as in step5_index_append */
  const float* ln_b;
  float ln_eps;
} step5_append_in;

/*
 * A decode step's indexer work in one call: step5_index_append of each
 * row's new token (as with STEP5_APPEND_ONE_PER_SEQ) and
 * step5_index_score_topk of the rows, with the same results as those two
 * calls made one after the other.
 * [TensorFold #903, indexer commit note: every completed region summarised;
 * q prep, scores, top 512; prompt-path commit note: the k and z rings]
 *
 * A row scores only regions before its own, and the append writes a row's
 * ring slot and, when the token completes it, the row's own region, so the
 * two halves touch different data when no two rows share a sequence: the
 * appends then run in extra workgroups of the selection's launch, on
 * compute units the selection leaves idle, instead of a launch of their own.
 * Precondition (device values, not checked): no two rows share a sequence,
 * as STEP5_APPEND_ONE_PER_SEQ guarantees for step5_index_append.
 *
 * ap          the append's own arguments (step5_append_in), not null.
 * flags, q .. ws_bytes, stream: as for step5_index_score_topk, except that
 *             rope_cs is required (the append's k prep uses it) and the
 *             summary is written (each completed region); ap and these
 *             arguments are checked as the two calls check theirs, and an
 *             error from either writes nothing.
 * rows == 0 is a successful no-op.
 */
int step5_index_append_score_topk(const step5_geom* geom, uint32_t flags,
                                  const step5_append_in* ap, const void* q, int64_t q_stride_row,
                                  const float* q_norm_w, float q_eps, const void* rope_cs,
                                  int64_t rope_rows, const float* w_head, int64_t w_stride_row,
                                  const int32_t* row_seq, const int64_t* row_pos, int32_t rows,
                                  void* summary, int64_t B, int64_t R_cap, int64_t s_stride_b,
                                  int32_t* sel_ids, float* sel_scores, void* workspace,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * Attention of each row over its selected regions plus its own region.
 * [TensorFold #903, indexer commit note: attention over the picks and the
 * row's own region; attention commit notes: keys split across workers whose
 * online-softmax states merge in a fixed order]
 *
 * q           bf16 [rows, q_heads, head_dim], after its rotation; row stride
 *             q_stride_row elements (a multiple of 8).
 * k_cache, v_cache
 *             bf16 [B, T_cap, kv_heads, head_dim]; element strides kv_stride_b
 *             and kv_stride_t (multiples of 8); a token's kv_heads*head_dim
 *             values contiguous.
 * sel_ids     int32 [rows, kv_heads, topk]: region ids per (row, KV head),
 *             -1 for none (as step5_index_score_topk writes them). Ids must be
 *             distinct; ids outside 0 .. floor(p/8)-1 are skipped.
 * row_seq, row_pos
 *             as above; p < T_cap.
 * softmax_scale
 *             finite and > 0 (1/sqrt(head_dim) for the Step-5 layer).
 * out         out: bf16 [rows, q_heads, head_dim], contiguous.
 * out_lse     out, nullable: fp32 [rows, q_heads]: natural-log sum of
 *             exp(scale * q.k) over the row's tokens.
 * workspace   device scratch of at least step5_sparse_attn_workspace() bytes,
 *             256-byte aligned (may be null when that is 0). It must be all
 *             zero before its first use by this call (it holds arrival
 *             counters as well as split states); every call leaves the
 *             counters zero again, so a workspace zeroed once can be reused by
 *             any number of calls, one at a time.
 * Query head h reads KV head h / (q_heads / kv_heads).
 * rows == 0 is a successful no-op.
 */
int step5_sparse_attn(const step5_geom* geom, const void* q, int64_t q_stride_row,
                      const void* k_cache, const void* v_cache, int64_t B, int64_t kv_stride_b,
                      int64_t kv_stride_t, int64_t T_cap, const int32_t* sel_ids,
                      const int32_t* row_seq, const int64_t* row_pos, int32_t rows,
                      float softmax_scale, void* out, float* out_lse, void* workspace,
                      size_t ws_bytes, hipStream_t stream);

/* Workspace bytes step5_sparse_attn needs for `rows` rows (0 if none is
 * needed or the geometry is not accepted). */
size_t step5_sparse_attn_workspace(const step5_geom* geom, int32_t rows);

/*
 * step5_sparse_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same arguments, results and kernels as step5_sparse_attn,
 * without the workspace arguments: the split states live in a device array
 * of the library, 16 MiB (STEP5_SPARSE_ATTN_STATIC_BYTES) per GPU, held from
 * the library's load until the process ends. The call allocates and frees
 * nothing; its first call on a device looks the array's address up once.
 * The array starts zero and every call leaves its counters zero. Calls
 * whose step5_sparse_attn_workspace() exceeds the array return
 * STEP5_E_WORKSPACE (no accepted geometry needs more than about 12.7 MB);
 * a stream that belongs to another device than the current one returns
 * STEP5_E_INVALID. Every call on one GPU uses the same array: calls that
 * overlap on one GPU (different streams, or different host threads) race
 * and must be ordered by the caller. Nothing in the array needs to start
 * at any other value.
 */
#define STEP5_SPARSE_ATTN_STATIC_BYTES ((size_t)16 << 20)
int step5_sparse_attn_noalloc(const step5_geom* geom, const void* q, int64_t q_stride_row,
                              const void* k_cache, const void* v_cache, int64_t B,
                              int64_t kv_stride_b, int64_t kv_stride_t, int64_t T_cap,
                              const int32_t* sel_ids, const int32_t* row_seq,
                              const int64_t* row_pos, int32_t rows, float softmax_scale,
                              void* out, float* out_lse, hipStream_t stream);

/*
 * The fused projection of a full-attention layer: one product of the normed
 * hidden state with a weight whose rows are the attention's q, k, v and the
 * indexer's q, k, z and gate rows, written straight into seven outputs.
 * [vLLM, "vllm.models.step5.nvidia.model", Step5FusedQKVIndexerLinear:
 * forward (one hidden @ W^T) and split_indexer]
 *
 * hidden      bf16 [rows, hidden_size], row stride hidden_stride_row
 *             elements (a multiple of 8); 16-byte aligned.
 * weight      bf16 [N, hidden_size], rows contiguous, 16-byte aligned;
 *             N = q_heads*head_dim + 2*kv_heads*head_dim + idx_heads*idx_dim
 *             + 2*groups*idx_dim + gate_size, its rows in the order of the
 *             outputs below.
 * gate_size   columns of the gate (0 or more, a multiple of 16; one per query
 *             head for the Step-5 layer: 16).
 * out         step5_proj_out[7], in the weight's row order: q [rows,
 *             q_heads*head_dim], k and v [rows, kv_heads*head_dim], index_q
 *             [rows, idx_heads*idx_dim], index_k and index_z [rows,
 *             groups*idx_dim], gate [rows, gate_size]; each bf16, 16-byte
 *             aligned, row stride stride_row elements (a multiple of 8, at
 *             least the part's width); a part of width 0 is not touched.
 * Each output element is the fp32 sum of the bf16 products over hidden_size,
 * rounded once to bf16 (nearest even). hidden_size must be a multiple of 128
 * (else STEP5_E_UNSUPPORTED). No workspace. rows == 0 is a successful no-op.
 */
typedef struct step5_proj_out {
  void* ptr;
  int64_t stride_row;
} step5_proj_out;

int step5_qkv_index_project(const step5_geom* geom, const void* hidden, int64_t hidden_stride_row,
                            int32_t rows, int32_t hidden_size, const void* weight,
                            int32_t gate_size, const step5_proj_out* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STEP5_H */
