// Internal launch interface between the C ABI (step5.cpp, argument checks and
// workspace carving) and the kernel files. Arguments arrive here already
// validated; the launchers only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace s5 {

struct SummarizeArgs {
  const void* k;
  const void* z;
  int64_t B, T, t0, sb, st;
  const float* ln_w;
  const float* ln_b;
  float eps;
  const void* rope;
  void* summary;
  int64_t ssb;
};
hipError_t launch_summarize(const SummarizeArgs& a, hipStream_t stream);

struct AppendArgs {
  const void* k_new;       // bf16 [rows, 4, 64], row stride new_stride_row (elements)
  const void* z_new;
  int64_t new_stride_row;
  const int32_t* row_seq;
  const int64_t* row_pos;
  int32_t rows;
  void* k_ring;            // bf16 [B, slots, 4, 64], sequence stride ring_stride_b (elements)
  void* z_ring;
  int64_t B, slots, ring_stride_b;
  const float* ln_w;
  const float* ln_b;
  float eps;
  const void* rope;
  int64_t rope_rows;
  void* summary;
  int64_t ssb, R_cap;
  bool one_per_seq;        // no two rows share a sequence: one fused launch
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

struct QPrepArgs {
  bool prepared;          // q is already e4m3 (row stride in bytes); else bf16 (elements)
  const void* q;
  int64_t q_stride_row;
  int32_t rows;
  const float* w;
  float eps;
  const void* rope;
  int64_t rope_rows;
  const int64_t* row_pos;
  uint8_t* q8;            // [rows, 16, 64] e4m3
  unsigned* arrivals;     // [rows*8]: top-k arrival counters (zeroed by the q prep or the
                          // exact scorer), then the exact path's survivor counts (zeroed
                          // by the exact scorer)
};
hipError_t launch_qprep(const QPrepArgs& a, hipStream_t stream);

struct ScoreArgs {
  const uint8_t* q8;      // from launch_qprep, [rows, 16, 64]
  int64_t q8_stride_row;  // bytes
  int32_t rows;
  const float* w_head;
  int64_t w_stride_row;
  const int32_t* row_seq;
  const int64_t* row_pos;
  const uint8_t* summary;
  int64_t B, R_cap, ssb;
  int64_t pos_limit;      // rows at p >= pos_limit are invalid (no rope row)
  bool exact;             // exact scores (score_exact_mode) instead of intervals; the exact
                          // kernel also does the q prep from `prep` (no launch_qprep)
  QPrepArgs prep;
  float2* bounds;         // [rows, 4, R_cap]: interval holding each exact score, or (exact)
                          // the exact scores as float [rows, 4, R_cap]
  uint32_t* pool;         // exact mode, several selection chunks: [rows*4, blocks, 8] keys
                          // for the selection's threshold (see topk_pool_bytes); else null
};
// Rows up to S5_EXACT_MAX_ROWS are scored exactly on the fp64 matrix cores,
// the query prep fused in; more rows get their query prepped by its own
// kernel, intervals from the bf16 matrix cores, and exact rescoring of the
// candidates that can reach each row's top 512.
#ifndef S5_EXACT_MAX_ROWS
#define S5_EXACT_MAX_ROWS 64
#endif
inline bool score_exact_mode(int32_t rows) { return rows <= S5_EXACT_MAX_ROWS; }
// Interval-mode batches whose units have at most 4,096 candidates (contexts
// up to 32K tokens: a prefill chunk) skip the score pass: the selection
// kernel computes each unit's intervals itself (no interval buffer).
#ifndef S5_FUSED_SELECT_MAX_RCAP
#define S5_FUSED_SELECT_MAX_RCAP 4096
#endif
inline bool select_fused(int32_t rows, int64_t R_cap) {
  return !score_exact_mode(rows) && R_cap <= S5_FUSED_SELECT_MAX_RCAP;
}
hipError_t launch_score(const ScoreArgs& a, hipStream_t stream);

// Top-k selection plan: the candidates of a (row, group) are cut into
// `nchunks` chunks of `chunk` candidates; with one chunk the selection is
// done in one pass, otherwise each chunk keeps its best 512 and a second
// pass picks the best 512 of their union.
struct TopkPlan {
  int64_t chunk;
  int32_t nchunks;
};
TopkPlan topk_plan(int32_t rows, int64_t R_cap);
size_t topk_partial_bytes(int32_t rows, int64_t R_cap);
// exact scores cut into several chunks: the scorer's threshold keys, 8 per
// (row, group) and block of 256 candidates (0 bytes otherwise)
size_t topk_pool_bytes(int32_t rows, int64_t R_cap);

struct TopkArgs {
  const float2* bounds;  // [rows, 4, R_cap] from launch_score
  bool exact;            // bounds holds exact scores (see ScoreArgs)
  bool fused;            // select_fused: no bounds; intervals computed from q8
  const uint8_t* q8;     // from launch_qprep, [rows, 16, 64] (intervals, rescoring)
  int64_t q8_stride_row; // bytes
  const float* w_head;
  int64_t w_stride_row;
  const uint8_t* summary;
  int64_t ssb;
  int32_t rows;
  int64_t R_cap;
  const int32_t* row_seq;
  const int64_t* row_pos;
  int64_t B;
  int64_t pos_limit;
  unsigned long long* partial;  // [rows*4, nchunks, 512] chunk lists when nchunks > 1
  const uint32_t* pool;  // exact with nchunks > 1: the scorer's threshold keys
  unsigned* arrivals;    // [rows*8]: arrival counters, then survivor counts; zero on
                         // entry (the q prep or the exact scorer zeroes them)
  int32_t* sel_ids;
  float* sel_scores;
  // optional: the cache append of a call whose rows are of distinct
  // sequences, run by extra workgroups of the same launch (one per row)
  const AppendArgs* append;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

// Attention plan: a (row, KV head) unit's 513 list entries (own region first,
// then the 512 selections) are cut into `nsplit` splits of `per_split`
// entries, each split one workgroup; several splits merge in a second pass.
struct AttnPlan {
  int32_t per_split;
  int32_t nsplit;
};
AttnPlan attn_plan(int32_t rows);
size_t attn_workspace_bytes(int32_t rows);
// the same for qpk query heads per KV head and a head dim of 128 or 192
size_t attn_mh_workspace_bytes(int32_t rows, int32_t qpk, int32_t head_dim);

struct AttnArgs {
  const void* q;
  int64_t q_stride_row;
  const void* k;
  const void* v;
  int64_t B, kv_sb, kv_st, T_cap;
  const int32_t* sel;
  const int32_t* row_seq;
  const int64_t* row_pos;
  int32_t rows;
  int32_t qpk;       // query heads per KV head (4, 8, 16)
  int32_t head_dim;  // 128 or 192
  float scale;
  void* out;
  float* lse;
  float* partial;
};
// qpk 4, head dim 128: attn_kernel (attn.hip); the rest: attn_mh_kernel (attn_mh.hip)
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);
// The split-state scratch of step5_sparse_attn_noalloc: a file-scope device
// array of kAttnStaticScratchBytes (attn.hip). attn_static_scratch gives its
// address on the stream's device (which must be the current device; else
// STEP5_E_INVALID), looked up once per device; STEP5_E_HIP if the lookup
// fails.
constexpr size_t kAttnStaticScratchBytes = (size_t)16 << 20;
int attn_static_scratch(hipStream_t stream, void** ptr);
hipError_t launch_attn_mh(const AttnArgs& a, hipStream_t stream);
// the context sweep over tiles of 32 rows for contexts below maxr regions
// (attn_tile.hip); tiles it does not take are left to attn_kernel
hipError_t launch_attn_tile(const AttnArgs& a, int32_t maxr, hipStream_t stream);
// merge of split states [rows*4 units][nsplit][qpk heads][m, l, o[head_dim]]
// into out and lse, in split order (attn_mh.hip)
hipError_t launch_attn_merge(const float* partial, int32_t nsplit, int32_t rows, int32_t qpk,
                             int32_t head_dim, void* out, float* lse, hipStream_t stream);

// Fused projection (proj.hip): hidden [rows, K] @ W[N, K]^T, the N output
// columns split over PROJ_PARTS outputs (part p: columns start[p] ..
// start[p+1]-1, every boundary a multiple of 16), bf16 with fp32 sums.
constexpr int PROJ_PARTS = 7;
struct ProjOuts {
  uint16_t* ptr[PROJ_PARTS];
  int64_t stride[PROJ_PARTS];  // elements between rows
  int32_t start[PROJ_PARTS + 1];
};
struct ProjArgs {
  const void* hidden;
  int64_t hidden_stride;
  int32_t rows;
  int32_t K;  // a multiple of 128
  const void* weight;  // bf16 [N, K], rows contiguous
  ProjOuts outs;
};
#ifndef S5_PROJ_WIDE_MIN_ROWS
#define S5_PROJ_WIDE_MIN_ROWS 256
#endif
hipError_t launch_proj(const ProjArgs& a, hipStream_t stream);

}  // namespace s5
