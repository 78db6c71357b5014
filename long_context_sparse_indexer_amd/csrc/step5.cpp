// C ABI of the Step-5 sparse-indexer path: argument checks, workspace
// layout, and the launch sequence of each call. Every host-checkable
// condition is checked before the first HIP call, so a rejected call enqueues
// nothing and writes nothing.
//
// Geometry rules: vLLM's Step-5 model page ("vllm.models.step5.nvidia.model",
// _validate_step5_dsa_parallel_geometry): indexer groups equal the attention
// KV heads, indexer heads divide into groups, 4/8/16 query heads per KV head.
#include <cmath>
#include <cstdint>

#include "step5.h"
#include "launch.hpp"

#define STEP5_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int32_t kIdxHeads = 16, kGroups = 4, kIdxDim = 64, kRopeDim = 32, kRegion = 8,
                  kTopk = 512, kKvHeads = 4;
constexpr int64_t kRegionBytes = (int64_t)kGroups * kIdxDim;  // e4m3 summary bytes per region
constexpr int64_t kMaxRcap = 524288;                            // 32 chunks of 16,384 candidates
constexpr int32_t kMaxScoreRows = 65535 * 4;                    // score grid: 4 rows per block row
constexpr size_t kAlign = 256;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_geom(const step5_geom* g) {
  if (!g) return STEP5_E_INVALID;
  if (g->idx_heads <= 0 || g->groups <= 0 || g->idx_dim <= 0 || g->rope_dim <= 0 ||
      g->region <= 0 || g->topk <= 0 || g->q_heads <= 0 || g->kv_heads <= 0 || g->head_dim <= 0)
    return STEP5_E_INVALID;
  if (g->groups != g->kv_heads) return STEP5_E_INVALID;
  if (g->idx_heads % g->groups) return STEP5_E_INVALID;
  if (g->q_heads % g->kv_heads) return STEP5_E_INVALID;
  const int32_t qpk = g->q_heads / g->kv_heads;
  if (qpk != 4 && qpk != 8 && qpk != 16) return STEP5_E_INVALID;
  if (g->rope_dim > g->idx_dim || (g->rope_dim & 1)) return STEP5_E_INVALID;
  if (g->idx_heads != kIdxHeads || g->groups != kGroups || g->idx_dim != kIdxDim ||
      g->rope_dim != kRopeDim || g->region != kRegion || g->topk != kTopk ||
      g->kv_heads != kKvHeads || (g->head_dim != 128 && g->head_dim != 192))
    return STEP5_E_UNSUPPORTED;
  return STEP5_OK;
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

struct ScoreWs {
  size_t q8 = 0, bounds = 0, partial = 0, pool = 0, arrivals = 0, total = 0;
};
ScoreWs score_ws(int32_t rows, int64_t R_cap) {
  ScoreWs w;
  size_t off = 0;
  w.q8 = off;   // prepared e4m3 query, [rows, idx_heads, idx_dim]
  off = up(off + (size_t)rows * kIdxHeads * kIdxDim);
  w.bounds = off;  // score interval per (row, group, candidate), unless fused
  if (!s5::select_fused(rows, R_cap))
    off = up(off + (size_t)rows * kGroups * (size_t)R_cap * 2 * sizeof(float));
  w.partial = off;  // chunk lists (or survivor lists) when units are cut into chunks
  off = up(off + s5::topk_partial_bytes(rows, R_cap));
  w.pool = off;     // exact path with chunks: the scorer's threshold keys
  off = up(off + s5::topk_pool_bytes(rows, R_cap));
  w.arrivals = off;  // chunk arrival counters, then survivor counts, per (row, group)
  off = up(off + (size_t)rows * kGroups * 2 * sizeof(unsigned));
  w.total = off;
  return w;
}

int from_hip(hipError_t e) { return e == hipSuccess ? STEP5_OK : STEP5_E_HIP; }

static_assert(s5::kAttnStaticScratchBytes == STEP5_SPARSE_ATTN_STATIC_BYTES,
              "the static attention scratch is the size the header states");

}  // namespace

STEP5_EXPORT const char* step5_status_str(int status) {
  switch (status) {
    case STEP5_OK: return "ok";
    case STEP5_E_INVALID: return "invalid argument";
    case STEP5_E_UNSUPPORTED: return "unsupported geometry or size";
    case STEP5_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case STEP5_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

STEP5_EXPORT int step5_index_summarize(const step5_geom* geom, const void* k, const void* z,
                                       int64_t B, int64_t T, int64_t t0, int64_t kz_stride_b,
                                       int64_t kz_stride_t, const float* ln_w, const float* ln_b,
                                       float ln_eps, const void* rope_cs, int64_t rope_rows,
                                       void* summary, int64_t s_stride_b, int64_t R_cap,
                                       hipStream_t stream) {
  const int gs = check_geom(geom);
  if (gs) return gs;
  if (B < 0 || T < 0 || t0 < 0 || (t0 % kRegion) != 0) return STEP5_E_INVALID;
  const int64_t nreg = T / kRegion;
  if (B == 0 || nreg == 0) return STEP5_OK;
  if (!k || !z || !ln_w || !ln_b || !rope_cs || !summary) return STEP5_E_INVALID;
  if (!aligned(k, 16) || !aligned(z, 16) || !aligned(ln_w, 16) || !aligned(ln_b, 16) ||
      !aligned(rope_cs, 16) || !aligned(summary, 16))
    return STEP5_E_INVALID;
  if (kz_stride_t < (int64_t)kGroups * kIdxDim || (kz_stride_t % 8) != 0) return STEP5_E_INVALID;
  if (kz_stride_b < 0 || (kz_stride_b % 8) != 0) return STEP5_E_INVALID;
  if (B > 1 && kz_stride_b < nreg * kRegion * kz_stride_t) return STEP5_E_INVALID;
  if (!finite_pos(ln_eps)) return STEP5_E_INVALID;
  if (rope_rows < t0 + nreg * kRegion) return STEP5_E_INVALID;
  if (R_cap < 1 || t0 / kRegion + nreg > R_cap) return STEP5_E_INVALID;
  if (s_stride_b < 0 || (s_stride_b % 16) != 0) return STEP5_E_INVALID;
  if (B > 1 && s_stride_b < R_cap * kRegionBytes) return STEP5_E_INVALID;

  s5::SummarizeArgs a;
  a.k = k;
  a.z = z;
  a.B = B;
  a.T = nreg * kRegion;
  a.t0 = t0;
  a.sb = kz_stride_b;
  a.st = kz_stride_t;
  a.ln_w = ln_w;
  a.ln_b = ln_b;
  a.eps = ln_eps;
  a.rope = rope_cs;
  a.summary = summary;
  a.ssb = s_stride_b;
  return from_hip(s5::launch_summarize(a, stream));
}

// Checks the arguments of an append and fills its launch arguments.
static int append_args(uint32_t flags, const void* k_new, const void* z_new,
                       int64_t new_stride_row, const int32_t* row_seq, const int64_t* row_pos,
                       int32_t rows, void* k_ring, void* z_ring, int64_t B, int64_t ring_slots,
                       int64_t ring_stride_b, const float* ln_w, const float* ln_b, float ln_eps,
                       const void* rope_cs, int64_t rope_rows, void* summary, int64_t s_stride_b,
                       int64_t R_cap, s5::AppendArgs* a) {
  if (rows < 0 || (flags & ~STEP5_APPEND_ONE_PER_SEQ) != 0) return STEP5_E_INVALID;
  if (rows == 0) return STEP5_OK;
  if (!k_new || !z_new || !row_seq || !row_pos || !k_ring || !z_ring || !ln_w || !ln_b ||
      !rope_cs || !summary)
    return STEP5_E_INVALID;
  if (!aligned(k_new, 16) || !aligned(z_new, 16) || !aligned(k_ring, 16) || !aligned(z_ring, 16) ||
      !aligned(ln_w, 16) || !aligned(ln_b, 16) || !aligned(rope_cs, 16) || !aligned(summary, 16) ||
      !aligned(row_seq, 4) || !aligned(row_pos, 8))
    return STEP5_E_INVALID;
  const int64_t tok = (int64_t)kGroups * kIdxDim;  // elements of one token's k (or z)
  if (new_stride_row < tok || (new_stride_row % 8) != 0) return STEP5_E_INVALID;
  if (B < 1 || ring_slots < kRegion || (ring_slots % kRegion) != 0) return STEP5_E_INVALID;
  if (ring_stride_b < 0 || (ring_stride_b % 8) != 0) return STEP5_E_INVALID;
  if (B > 1 && ring_stride_b < ring_slots * tok) return STEP5_E_INVALID;
  if (!finite_pos(ln_eps) || rope_rows < kRegion) return STEP5_E_INVALID;
  if (R_cap < 1 || s_stride_b < 0 || (s_stride_b % 16) != 0) return STEP5_E_INVALID;
  if (B > 1 && s_stride_b < R_cap * kRegionBytes) return STEP5_E_INVALID;
  a->k_new = k_new;
  a->z_new = z_new;
  a->new_stride_row = new_stride_row;
  a->row_seq = row_seq;
  a->row_pos = row_pos;
  a->rows = rows;
  a->k_ring = k_ring;
  a->z_ring = z_ring;
  a->B = B;
  a->slots = ring_slots;
  a->ring_stride_b = ring_stride_b;
  a->ln_w = ln_w;
  a->ln_b = ln_b;
  a->eps = ln_eps;
  a->rope = rope_cs;
  a->rope_rows = rope_rows;
  a->summary = summary;
  a->ssb = s_stride_b;
  a->R_cap = R_cap;
  a->one_per_seq = (flags & STEP5_APPEND_ONE_PER_SEQ) != 0;
  return STEP5_OK;
}

STEP5_EXPORT int step5_index_append(const step5_geom* geom, uint32_t flags, const void* k_new,
                                    const void* z_new,
                                    int64_t new_stride_row, const int32_t* row_seq,
                                    const int64_t* row_pos, int32_t rows, void* k_ring,
                                    void* z_ring, int64_t B, int64_t ring_slots,
                                    int64_t ring_stride_b, const float* ln_w, const float* ln_b,
                                    float ln_eps, const void* rope_cs, int64_t rope_rows,
                                    void* summary, int64_t s_stride_b, int64_t R_cap,
                                    hipStream_t stream) {
  const int gs = check_geom(geom);
  if (gs) return gs;
  s5::AppendArgs a;
  const int st = append_args(flags, k_new, z_new, new_stride_row, row_seq, row_pos, rows, k_ring,
                             z_ring, B, ring_slots, ring_stride_b, ln_w, ln_b, ln_eps, rope_cs,
                             rope_rows, summary, s_stride_b, R_cap, &a);
  if (st || rows == 0) return st;
  return from_hip(s5::launch_append(a, stream));
}

STEP5_EXPORT size_t step5_index_score_topk_workspace(const step5_geom* geom, int32_t rows,
                                                     int64_t R_cap) {
  if (check_geom(geom) || rows < 0 || rows > kMaxScoreRows || R_cap < 1 || R_cap > kMaxRcap)
    return 0;
  if (rows == 0) return 0;
  return score_ws(rows, R_cap).total;
}

// score_topk; with `ap`, the selection launch also runs that append (rows of
// distinct sequences, checked by the caller).
static int score_topk(const step5_geom* geom, uint32_t flags, const void* q, int64_t q_stride_row,
                      const float* q_norm_w, float q_eps, const void* rope_cs, int64_t rope_rows,
                      const float* w_head, int64_t w_stride_row, const int32_t* row_seq,
                      const int64_t* row_pos, int32_t rows, const void* summary, int64_t B,
                      int64_t R_cap, int64_t s_stride_b, int32_t* sel_ids, float* sel_scores,
                      void* workspace, size_t ws_bytes, const s5::AppendArgs* ap,
                      hipStream_t stream) {
  const int gs = check_geom(geom);
  if (gs) return gs;
  if (flags & ~STEP5_Q_E4M3) return STEP5_E_INVALID;
  if (rows < 0) return STEP5_E_INVALID;
  if (rows == 0) return STEP5_OK;
  if (rows > kMaxScoreRows) return STEP5_E_UNSUPPORTED;
  const bool q_ready = (flags & STEP5_Q_E4M3) != 0;
  if (!q || !aligned(q, 16)) return STEP5_E_INVALID;
  if (q_ready) {
    if (q_stride_row < (int64_t)kIdxHeads * kIdxDim || (q_stride_row % 16) != 0)
      return STEP5_E_INVALID;
  } else {
    if (q_stride_row < (int64_t)kIdxHeads * kIdxDim || (q_stride_row % 8) != 0)
      return STEP5_E_INVALID;
    if (!q_norm_w || !aligned(q_norm_w, 16) || !finite_pos(q_eps)) return STEP5_E_INVALID;
    if (!rope_cs || !aligned(rope_cs, 16) || rope_rows < 1) return STEP5_E_INVALID;
  }
  if (!w_head || !aligned(w_head, 4)) return STEP5_E_INVALID;
  if (w_stride_row != 0 && w_stride_row < kIdxHeads) return STEP5_E_INVALID;
  if (!row_seq || !row_pos || !aligned(row_seq, 4) || !aligned(row_pos, 8)) return STEP5_E_INVALID;
  if (!summary || !aligned(summary, 16)) return STEP5_E_INVALID;
  if (B < 1 || R_cap < 1) return STEP5_E_INVALID;
  if (R_cap > kMaxRcap) return STEP5_E_UNSUPPORTED;
  if (s_stride_b < 0 || (s_stride_b % 16) != 0) return STEP5_E_INVALID;
  if (B > 1 && s_stride_b < R_cap * kRegionBytes) return STEP5_E_INVALID;
  if (!sel_ids || !aligned(sel_ids, 4) || (sel_scores && !aligned(sel_scores, 4)))
    return STEP5_E_INVALID;
  const ScoreWs w = score_ws(rows, R_cap);
  if (ws_bytes < w.total || !workspace || !aligned(workspace, kAlign)) return STEP5_E_WORKSPACE;

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint8_t* q8 = ws + w.q8;
  s5::QPrepArgs qa;
  qa.prepared = q_ready;
  qa.q = q;
  qa.q_stride_row = q_stride_row;
  qa.rows = rows;
  qa.w = q_norm_w;
  qa.eps = q_eps;
  qa.rope = rope_cs;
  qa.rope_rows = q_ready ? 0 : rope_rows;
  qa.row_pos = row_pos;
  qa.q8 = q8;
  qa.arrivals = reinterpret_cast<unsigned*>(ws + w.arrivals);
  const bool exact = s5::score_exact_mode(rows);
  int st = exact ? STEP5_OK : from_hip(s5::launch_qprep(qa, stream));
  if (st) return st;
  s5::ScoreArgs sa;
  sa.prep = qa;
  sa.q8 = q8;
  sa.q8_stride_row = (int64_t)kIdxHeads * kIdxDim;
  sa.rows = rows;
  sa.w_head = w_head;
  sa.w_stride_row = w_stride_row;
  sa.row_seq = row_seq;
  sa.row_pos = row_pos;
  sa.summary = static_cast<const uint8_t*>(summary);
  sa.B = B;
  sa.R_cap = R_cap;
  sa.ssb = s_stride_b;
  sa.pos_limit = q_ready ? INT64_MAX : rope_rows;
  sa.exact = exact;
  sa.bounds = reinterpret_cast<float2*>(ws + w.bounds);
  sa.pool = s5::topk_pool_bytes(rows, R_cap) ? reinterpret_cast<uint32_t*>(ws + w.pool) : nullptr;
  const bool fused = s5::select_fused(rows, R_cap);
  if (!fused) {
    st = from_hip(s5::launch_score(sa, stream));
    if (st) return st;
  }
  s5::TopkArgs ta;
  ta.bounds = sa.bounds;
  ta.exact = sa.exact;
  ta.fused = fused;
  ta.q8 = q8;
  ta.q8_stride_row = sa.q8_stride_row;
  ta.w_head = w_head;
  ta.w_stride_row = w_stride_row;
  ta.summary = static_cast<const uint8_t*>(summary);
  ta.ssb = s_stride_b;
  ta.rows = rows;
  ta.R_cap = R_cap;
  ta.row_seq = row_seq;
  ta.row_pos = row_pos;
  ta.B = B;
  ta.pos_limit = sa.pos_limit;
  ta.partial = reinterpret_cast<unsigned long long*>(ws + w.partial);
  ta.pool = sa.pool;
  ta.arrivals = qa.arrivals;
  ta.sel_ids = sel_ids;
  ta.sel_scores = sel_scores;
  ta.append = ap;
  return from_hip(s5::launch_topk(ta, stream));
}

STEP5_EXPORT int step5_index_score_topk(const step5_geom* geom, uint32_t flags, const void* q,
                                        int64_t q_stride_row, const float* q_norm_w, float q_eps,
                                        const void* rope_cs, int64_t rope_rows,
                                        const float* w_head, int64_t w_stride_row,
                                        const int32_t* row_seq, const int64_t* row_pos,
                                        int32_t rows, const void* summary, int64_t B,
                                        int64_t R_cap, int64_t s_stride_b, int32_t* sel_ids,
                                        float* sel_scores, void* workspace, size_t ws_bytes,
                                        hipStream_t stream) {
  return score_topk(geom, flags, q, q_stride_row, q_norm_w, q_eps, rope_cs, rope_rows, w_head,
                    w_stride_row, row_seq, row_pos, rows, summary, B, R_cap, s_stride_b, sel_ids,
                    sel_scores, workspace, ws_bytes, nullptr, stream);
}

STEP5_EXPORT int step5_index_append_score_topk(
    const step5_geom* geom, uint32_t flags, const step5_append_in* ap, const void* q,
    int64_t q_stride_row, const float* q_norm_w, float q_eps, const void* rope_cs,
    int64_t rope_rows, const float* w_head, int64_t w_stride_row, const int32_t* row_seq,
    const int64_t* row_pos, int32_t rows, void* summary, int64_t B, int64_t R_cap,
    int64_t s_stride_b, int32_t* sel_ids, float* sel_scores, void* workspace, size_t ws_bytes,
    hipStream_t stream) {
  const int gs = check_geom(geom);
  if (gs) return gs;
  if (!ap) return STEP5_E_INVALID;
  s5::AppendArgs a;
  int st = append_args(STEP5_APPEND_ONE_PER_SEQ, ap->k_new, ap->z_new, ap->new_stride_row, row_seq,
                       row_pos, rows, ap->k_ring, ap->z_ring, B, ap->ring_slots,
                       ap->ring_stride_b, ap->ln_w, ap->ln_b, ap->ln_eps, rope_cs, rope_rows,
                       summary, s_stride_b, R_cap, &a);
  if (st) return st;
  return score_topk(geom, flags, q, q_stride_row, q_norm_w, q_eps, rope_cs, rope_rows, w_head,
                    w_stride_row, row_seq, row_pos, rows, summary, B, R_cap, s_stride_b, sel_ids,
                    sel_scores, workspace, ws_bytes, &a, stream);
}

STEP5_EXPORT size_t step5_sparse_attn_workspace(const step5_geom* geom, int32_t rows) {
  if (check_geom(geom) || rows <= 0 || rows > (INT32_MAX / 4)) return 0;
  const int32_t qpk = geom->q_heads / geom->kv_heads;
  const size_t b = (qpk == 4 && geom->head_dim == 128)
                       ? s5::attn_workspace_bytes(rows)
                       : s5::attn_mh_workspace_bytes(rows, qpk, geom->head_dim);
  return b ? up(b) : 0;
}

// Checks the arguments of a sparse-attention call (all but the workspace) and
// fills its launch arguments.
static int attn_args(const step5_geom* geom, const void* q, int64_t q_stride_row,
                     const void* k_cache, const void* v_cache, int64_t B, int64_t kv_stride_b,
                     int64_t kv_stride_t, int64_t T_cap, const int32_t* sel_ids,
                     const int32_t* row_seq, const int64_t* row_pos, int32_t rows,
                     float softmax_scale, void* out, float* out_lse, s5::AttnArgs* a) {
  const int gs = check_geom(geom);
  if (gs) return gs;
  if (rows < 0) return STEP5_E_INVALID;
  if (rows == 0) return STEP5_OK;
  if (rows > INT32_MAX / 4) return STEP5_E_UNSUPPORTED;
  const int64_t hd = geom->head_dim;
  if (!q || !aligned(q, 16) || q_stride_row < (int64_t)geom->q_heads * hd || (q_stride_row % 8))
    return STEP5_E_INVALID;
  if (!k_cache || !v_cache || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return STEP5_E_INVALID;
  if (B < 1 || T_cap < 1) return STEP5_E_INVALID;
  if (kv_stride_t < (int64_t)kKvHeads * hd || (kv_stride_t % 8)) return STEP5_E_INVALID;
  if (kv_stride_b < 0 || (kv_stride_b % 8)) return STEP5_E_INVALID;
  if (B > 1 && kv_stride_b < T_cap * kv_stride_t) return STEP5_E_INVALID;
  if (!sel_ids || !aligned(sel_ids, 4)) return STEP5_E_INVALID;
  if (!row_seq || !row_pos || !aligned(row_seq, 4) || !aligned(row_pos, 8)) return STEP5_E_INVALID;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.0f)) return STEP5_E_INVALID;
  if (!out || !aligned(out, 16) || (out_lse && !aligned(out_lse, 4))) return STEP5_E_INVALID;
  a->q = q;
  a->q_stride_row = q_stride_row;
  a->k = k_cache;
  a->v = v_cache;
  a->B = B;
  a->kv_sb = kv_stride_b;
  a->kv_st = kv_stride_t;
  a->T_cap = T_cap;
  a->sel = sel_ids;
  a->row_seq = row_seq;
  a->row_pos = row_pos;
  a->rows = rows;
  a->qpk = geom->q_heads / geom->kv_heads;
  a->head_dim = geom->head_dim;
  a->scale = softmax_scale;
  a->out = out;
  a->lse = out_lse;
  a->partial = nullptr;
  return STEP5_OK;
}

STEP5_EXPORT int step5_sparse_attn(const step5_geom* geom, const void* q, int64_t q_stride_row,
                                   const void* k_cache, const void* v_cache, int64_t B,
                                   int64_t kv_stride_b, int64_t kv_stride_t, int64_t T_cap,
                                   const int32_t* sel_ids, const int32_t* row_seq,
                                   const int64_t* row_pos, int32_t rows, float softmax_scale,
                                   void* out, float* out_lse, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  s5::AttnArgs a;
  const int st = attn_args(geom, q, q_stride_row, k_cache, v_cache, B, kv_stride_b, kv_stride_t,
                           T_cap, sel_ids, row_seq, row_pos, rows, softmax_scale, out, out_lse, &a);
  if (st || rows == 0) return st;
  const size_t need = step5_sparse_attn_workspace(geom, rows);
  if (ws_bytes < need || (need && (!workspace || !aligned(workspace, kAlign))))
    return STEP5_E_WORKSPACE;
  a.partial = static_cast<float*>(workspace);
  return from_hip(s5::launch_attn(a, stream));
}

STEP5_EXPORT int step5_sparse_attn_noalloc(const step5_geom* geom, const void* q,
                                           int64_t q_stride_row, const void* k_cache,
                                           const void* v_cache, int64_t B, int64_t kv_stride_b,
                                           int64_t kv_stride_t, int64_t T_cap,
                                           const int32_t* sel_ids, const int32_t* row_seq,
                                           const int64_t* row_pos, int32_t rows,
                                           float softmax_scale, void* out, float* out_lse,
                                           hipStream_t stream) {
  s5::AttnArgs a;
  const int st = attn_args(geom, q, q_stride_row, k_cache, v_cache, B, kv_stride_b, kv_stride_t,
                           T_cap, sel_ids, row_seq, row_pos, rows, softmax_scale, out, out_lse, &a);
  if (st || rows == 0) return st;
  const size_t need = step5_sparse_attn_workspace(geom, rows);
  if (need > s5::kAttnStaticScratchBytes) return STEP5_E_WORKSPACE;
  if (need) {
    void* scratch = nullptr;
    const int sst = s5::attn_static_scratch(stream, &scratch);
    if (sst) return sst;
    a.partial = static_cast<float*>(scratch);
  }
  return from_hip(s5::launch_attn(a, stream));
}

STEP5_EXPORT int step5_qkv_index_project(const step5_geom* geom, const void* hidden,
                                         int64_t hidden_stride_row, int32_t rows,
                                         int32_t hidden_size, const void* weight, int32_t gate_size,
                                         const step5_proj_out* out, hipStream_t stream) {
  const int gs = check_geom(geom);
  if (gs) return gs;
  if (rows < 0 || hidden_size <= 0 || gate_size < 0) return STEP5_E_INVALID;
  if (!hidden || !aligned(hidden, 16) || hidden_stride_row < hidden_size || (hidden_stride_row % 8))
    return STEP5_E_INVALID;
  if (!weight || !aligned(weight, 16) || !out) return STEP5_E_INVALID;
  if ((hidden_size % 128) || (gate_size % 16) || rows > 65535 * 16) return STEP5_E_UNSUPPORTED;
  const int64_t width[s5::PROJ_PARTS] = {
      (int64_t)geom->q_heads * geom->head_dim, (int64_t)geom->kv_heads * geom->head_dim,
      (int64_t)geom->kv_heads * geom->head_dim, (int64_t)geom->idx_heads * geom->idx_dim,
      (int64_t)geom->groups * geom->idx_dim,    (int64_t)geom->groups * geom->idx_dim,
      gate_size};
  s5::ProjArgs a;
  a.outs.start[0] = 0;
  for (int p = 0; p < s5::PROJ_PARTS; ++p) {
    const step5_proj_out& o = out[p];
    if (width[p] > 0 && (!o.ptr || !aligned(o.ptr, 16) || o.stride_row < width[p] ||
                         (o.stride_row % 8)))
      return STEP5_E_INVALID;
    a.outs.ptr[p] = static_cast<uint16_t*>(o.ptr);
    a.outs.stride[p] = o.stride_row;
    a.outs.start[p + 1] = a.outs.start[p] + (int32_t)width[p];
  }
  if (rows == 0) return STEP5_OK;
  a.hidden = hidden;
  a.hidden_stride = hidden_stride_row;
  a.rows = rows;
  a.K = hidden_size;
  a.weight = weight;
  return from_hip(s5::launch_proj(a, stream));
}
