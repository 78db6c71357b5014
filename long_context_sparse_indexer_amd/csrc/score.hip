// Indexer query prep and region scoring.
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// the indexer q has 16 heads, RMSNorm with scale (1 + w) and NEOX rotation of
// dims 0..31; a region's score for a KV group is the sum over the group's
// heads of relu(e4m3(q_h) . summary) * w_h.
//
// q prep rounding points (fp32): ms = sum64(x*x)/64, r = 1/sqrt(ms + eps),
// y = (x*r)*(1 + w), rotation a*c - b*s | b*c + a*s from bf16 cos/sin, bf16,
// then e4m3.
//
// Scoring is an fp8 x fp8 contraction over the 64 dims, done with the
// 16x16x32 fp8 MFMA (two per 64-dim dot, fp32 accumulation). Operand lanes:
// lane l = 16*q + n holds row/column n and the 16 contiguous bytes 16q..16q+15
// of the 64-byte vector; the first MFMA takes bytes 0..7 of each lane's slice
// and the second bytes 8..15, identically for both operands, so the pair
// covers each of the 64 products once. Output lane (n, q) holds column n,
// rows 4q..4q+3.
//
// Two tilings, chosen per block of 4 rows at run time:
//  - rows sharing one sequence (a prefill chunk): A = 4 rows x the 4 heads of
//    group g (16 MFMA rows), B = 16 candidates of group g: every MFMA output
//    is used, and each summary byte loaded serves 4 rows;
//  - rows of different sequences (decode): per row, A = its 16 heads,
//    B = 4 candidates x 4 groups (1 KB contiguous); only the lanes whose head
//    group matches the column's group are kept. Decode scoring is bound by
//    the summary stream, not by the matrix cores.
// Epilogue per (row, group, candidate): t_h = max(dot_h, +0), then
// ((t0*w0 + t1*w1) + t2*w2) + t3*w3 with separately rounded products.
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

// ---------------------------------------------------------------------------
// q prep: one 8-lane group per (row, head); lane c holds dims 8c..8c+7.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qprep_kernel(const uint16_t* __restrict__ q, int64_t qs,
                                                    int32_t rows, const float* __restrict__ w,
                                                    float eps, const uint16_t* __restrict__ rope,
                                                    int64_t rope_rows,
                                                    const int64_t* __restrict__ row_pos,
                                                    uint8_t* __restrict__ q8) {
  const int lane = threadIdx.x & 63;
  const int c = threadIdx.x & 7;
  const int64_t vec = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  if (vec >= (int64_t)rows * 16) return;  // whole 8-lane groups leave together
  const int64_t r = vec >> 4;
  const int h = (int)(vec & 15);
  int64_t p = row_pos[r];
  if (p < 0 || p >= rope_rows) p = 0;  // such a row selects nothing later; keep reads in range

  float x[8], sq[8], y[8];
  unpack_bf16x8(ldg16(q + r * qs + h * 64 + c * 8), x);
#pragma unroll
  for (int i = 0; i < 8; ++i) sq[i] = x[i] * x[i];
  const float ms = sum8_lanes(pair8(sq), lane) / 64.0f;
  const float rr = 1.0f / sqrtf(ms + eps);
  const float4 w0 = reinterpret_cast<const float4*>(w)[2 * c];
  const float4 w1 = reinterpret_cast<const float4*>(w)[2 * c + 1];
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float scale = 1.0f + wv[i];
    y[i] = (x[i] * rr) * scale;
  }
  const bool rotated = c < 4, first_half = c < 2;
  const int fi = (c & 1) * 8;
  float cf[8], sf[8];
  unpack_bf16x8(ldg16(rope + p * 32 + fi), cf);
  unpack_bf16x8(ldg16(rope + p * 32 + 16 + fi), sf);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float other = dpp<DPP_QUAD_XOR2>(y[i]);
    const float own_c = y[i] * cf[i];
    const float oth_s = other * sf[i];
    const float rot = first_half ? (own_c - oth_s) : (own_c + oth_s);
    const uint32_t code = e4m3_from_bf16(bf16_bits(rotated ? rot : y[i]));
    if (i < 4) lo |= code << (8 * i);
    else hi |= code << (8 * (i - 4));
  }
  *reinterpret_cast<uint2*>(q8 + vec * 64 + c * 8) = make_uint2(lo, hi);
}

hipError_t launch_qprep(const QPrepArgs& a, hipStream_t stream) {
  const int64_t vecs = (int64_t)a.rows * 16;
  if (vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)((vecs + 31) / 32)), dim3(256), 0, stream,
                     (const uint16_t*)a.q, a.q_stride_row, a.rows, a.w, a.eps,
                     (const uint16_t*)a.rope, a.rope_rows, a.row_pos, a.q8);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------
constexpr int SC_CB = 256;  // candidates per block

__device__ inline long lo8(uint4 v) { return (long)(((unsigned long)v.y << 32) | v.x); }
__device__ inline long hi8(uint4 v) { return (long)(((unsigned long)v.w << 32) | v.z); }

__device__ inline f32x4 dot64(uint4 a, uint4 b) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(lo8(a), lo8(b), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(hi8(a), hi8(b), acc, 0, 0, 0);
  return acc;
}

__device__ inline float relu0(float v) { return v > 0.0f ? v : 0.0f; }

__device__ inline float group_score(f32x4 d, const float* __restrict__ w4) {
  const float t0 = relu0(d[0]) * w4[0];
  const float t1 = relu0(d[1]) * w4[1];
  const float t2 = relu0(d[2]) * w4[2];
  const float t3 = relu0(d[3]) * w4[3];
  float s = t0 + t1;
  s = s + t2;
  s = s + t3;
  return s;
}

__global__ __launch_bounds__(256) void score_kernel(
    const uint8_t* __restrict__ q8, int64_t qs8, int32_t rows, const float* __restrict__ w_head,
    int64_t w_stride, const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos,
    const uint8_t* __restrict__ S, int64_t B, int64_t R_cap, int64_t ssb, int64_t pos_limit,
    float* __restrict__ scores) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int r0 = blockIdx.y * 4;
  const int64_t cb0 = (int64_t)blockIdx.x * SC_CB;
  const int nr = min(4, rows - r0);

  int32_t seq[4];
  int64_t ncand[4];
  int64_t maxc = 0;
  bool shared = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    seq[i] = -1;
    ncand[i] = 0;
    if (i < nr) {
      const int32_t s = row_seq[r0 + i];
      const int64_t p = row_pos[r0 + i];
      const bool ok = s >= 0 && s < B && p >= 0 && p < pos_limit && (p >> 3) <= R_cap;
      seq[i] = ok ? s : -1;
      ncand[i] = ok ? (p >> 3) : 0;
      maxc = ncand[i] > maxc ? ncand[i] : maxc;
    }
  }
  if (cb0 >= maxc) return;
  int32_t s0 = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (seq[i] >= 0) {
      if (s0 < 0) s0 = seq[i];
      else if (seq[i] != s0) shared = false;
    }
  }

  if (shared) {
    // ---- one sequence: A = (4 rows x 4 heads of group g), B = 16 candidates of g
    const uint8_t* Sb = S + (int64_t)s0 * ssb;
    const int rr = n >> 2, hh = n & 3;
    uint4 aq[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      aq[g] = make_uint4(0, 0, 0, 0);
      if (rr < nr && seq[rr] >= 0) aq[g] = ldg16(q8 + (int64_t)(r0 + rr) * qs8 + (4 * g + hh) * 64 + 16 * qd);
    }
    // this lane's output row (rows 4qd..4qd+3 of the MFMA = row qd of the tile)
    const int orow = r0 + qd;
    const bool orow_ok = qd < nr && seq[qd] >= 0;
    const int64_t onc = orow_ok ? ncand[qd] : 0;
    float w4[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[g][i] = orow_ok ? w_head[(int64_t)orow * w_stride + 4 * g + i] : 0.f;

    const int64_t jw = cb0 + wave * 64;
    uint4 bq[4][4];
#pragma unroll
    for (int stl = 0; stl < 4; ++stl) {
      const int64_t j = jw + stl * 16 + n;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bq[stl][g] = (j < maxc) ? ldg16(Sb + j * 256 + g * 64 + 16 * qd) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int stl = 0; stl < 4; ++stl) {
      const int64_t j = jw + stl * 16 + n;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d = dot64(aq[g], bq[stl][g]);
        if (j < onc) scores[((int64_t)orow * 4 + g) * R_cap + j] = group_score(d, w4[g]);
      }
    }
  } else {
    // ---- rows of different sequences: wave w scores row r0 + w
    if (wave >= nr || seq[wave] < 0) return;
    const int row = r0 + wave;
    const int64_t nc = ncand[wave];
    if (cb0 >= nc) return;
    const uint8_t* Sb = S + (int64_t)seq[wave] * ssb;
    const uint4 aq = ldg16(q8 + (int64_t)row * qs8 + n * 64 + 16 * qd);
    float w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w4[i] = w_head[(int64_t)row * w_stride + 4 * qd + i];
    const bool keep = qd == (n & 3);
    const int64_t jend = (cb0 + SC_CB < nc) ? cb0 + SC_CB : nc;
    for (int64_t jb = cb0; jb < jend; jb += 32) {
      uint4 bq[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = jb + u * 4 + (n >> 2);
        bq[u] = (j < jend) ? ldg16(Sb + (jb + u * 4) * 256 + n * 64 + 16 * qd) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = jb + u * 4 + (n >> 2);
        const f32x4 d = dot64(aq, bq[u]);
        if (keep && j < jend) scores[((int64_t)row * 4 + qd) * R_cap + j] = group_score(d, w4);
      }
    }
  }
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.rows == 0 || a.R_cap == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.R_cap + SC_CB - 1) / SC_CB), (unsigned)((a.rows + 3) / 4));
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, stream, a.q8, a.q8_stride_row, a.rows,
                     a.w_head, a.w_stride_row, a.row_seq, a.row_pos, a.summary, a.B, a.R_cap,
                     a.ssb, a.pos_limit, a.scores);
  return hipGetLastError();
}

}  // namespace s5
