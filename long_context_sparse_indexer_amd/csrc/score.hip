// Indexer query prep and region scoring (bounds).
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// the indexer q has 16 heads, RMSNorm with scale (1 + w) and NEOX rotation of
// dims 0..31; a region's score for a KV group is the sum over the group's
// heads of relu(e4m3(q_h) . summary) * w_h; the top 512 by (-score, id) are
// kept in that order.
//
// q prep rounding points (fp32): ms = sum64(x*x)/64, r = 1/sqrt(ms + eps),
// y = (x*r)*(1 + w), rotation a*c - b*s | b*c + a*s from bf16 cos/sin, bf16,
// then e4m3. It writes the e4m3 query (for the matrix cores) and its exact
// fp64 values laid out [row][group][dim][4 heads] (for exact rescoring).
//
// Scoring is a 64-dim contraction of e4m3 vectors, run on the matrix cores:
// every e4m3 value is exactly a bf16 value, so the operands are widened in
// registers (hardware fp8 -> fp32 conversion, keep the high half) and fed to
// the 16x16x32 bf16 MFMA, two per dot, fp32 accumulation. (Measured on
// gfx950: the fp8 MFMA's accumulation loses up to 2^-10.8 of sum |q s|,
// while the bf16 MFMA on the same values stays within 2^-21.8 of it and
// returns the correctly rounded exact dot for normal and heavy-tailed data.)
// Accumulation can still round, and scores of 10^4..10^5 candidates can be a
// few ulps apart, so the kernel emits an interval that holds the exact score:
// the same MFMA on absolute values (sign bits cleared) gives A = sum |q s|,
// and with delta = 2^-18 * sum_h |w_h| A_h + 2^-22 |s~| the exact score lies
// in [s~ - delta, s~ + delta] (a margin of 4 over eight truncating additions
// per dot, 14 over the measured worst case). The selection pass uses the
// intervals to find which candidates can reach the top 512 and rescores only
// those exactly (exact.hpp), so exactness never rests on the accumulator.
//
// With few rows (decode) the intervals cost more than they save: there every
// candidate is scored exactly on the fp64 matrix cores instead
// (score_exact_mfma_kernel) and the selection pass reads plain scores.
//
// Operand lanes: lane l = 16q + n holds row/column n and the 16 contiguous
// e4m3 bytes 16q..16q+15 of the 64-byte vector, widened to 16 bf16; the first
// MFMA takes elements 0..7 of each lane's slice and the second 8..15,
// identically for both operands. Output lane (n, q) holds column n, rows
// 4q..4q+3.
//
// Two tilings, chosen per block of 4 rows at run time:
//  - rows sharing one sequence (a prefill chunk): A = 4 rows x the 4 heads of
//    group g (16 MFMA rows), B = 16 candidates of group g: every output is
//    used and each summary byte loaded serves 4 rows;
//  - rows of different sequences (decode): per row, A = its 16 heads,
//    B = 4 candidates x 4 groups (1 KB contiguous); lanes whose head group
//    matches the column's group keep their result.
#include "device.hpp"
#include "exact.hpp"
#include "interval.hpp"
#include "launch.hpp"

namespace s5 {

// ---------------------------------------------------------------------------
// q prep of one (row r, head h) by an 8-lane group: lane c gets the e4m3
// codes of dims 8c..8c+7, packed (byte i = dim 8c + i; all 8 lanes of the
// group must be active).
// mode 0: bf16 input, RMSNorm with scale (1 + w), rotation, bf16, e4m3;
// mode 1: the input is already e4m3.
// The bf16 and e4m3 roundings use gfx950's conversion instructions
// (bf16x2_hw, e4m3x2_hw), which give the same bits as the software forms.
// ---------------------------------------------------------------------------
// The bf16 path in two halves, so that a caller can issue the loads first
// and keep other loads in flight while they arrive: qprep8_load reads dims
// 8c..8c+7 of head h of row r, the rotation's cos and sin at position p
// (already clamped to the table) and the norm weights; qprep8_math does the
// arithmetic.
struct QPrep8In {
  uint4 q, c, s;
  float4 w0, w1;
};
__device__ inline QPrep8In qprep8_load(const uint16_t* __restrict__ q, int64_t qs, int64_t r, int h,
                                       int c, const float* __restrict__ w,
                                       const uint16_t* __restrict__ rope, int64_t p) {
  const int fi = (c & 1) * 8;
  QPrep8In in;
  in.q = ldg16(q + r * qs + h * 64 + c * 8);
  in.c = ldg16(rope + p * 32 + fi);
  in.s = ldg16(rope + p * 32 + 16 + fi);
  in.w0 = reinterpret_cast<const float4*>(w)[2 * c];
  in.w1 = reinterpret_cast<const float4*>(w)[2 * c + 1];
  return in;
}

__device__ inline uint2 qprep8_math(const QPrep8In& in, int c, int lane, float eps) {
  const bool rotated = c < 4, first_half = c < 2;
  float x[8], sq[8], y[8];
  unpack_bf16x8(in.q, x);
#pragma unroll
  for (int i = 0; i < 8; ++i) sq[i] = x[i] * x[i];
  const float ms = sum8_lanes(pair8(sq), lane) / 64.0f;
  const float rr = 1.0f / sqrtf(ms + eps);
  const float wv[8] = {in.w0.x, in.w0.y, in.w0.z, in.w0.w, in.w1.x, in.w1.y, in.w1.z, in.w1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float scale = 1.0f + wv[i];
    y[i] = (x[i] * rr) * scale;
  }
  float cf[8], sf[8], v[8];
  unpack_bf16x8(in.c, cf);
  unpack_bf16x8(in.s, sf);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float other = dpp<DPP_QUAD_XOR2>(y[i]);
    const float own_c = y[i] * cf[i];
    const float oth_s = other * sf[i];
    const float rot = first_half ? (own_c - oth_s) : (own_c + oth_s);
    v[i] = rotated ? rot : y[i];
  }
  float bf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t pk = bf16x2_hw(v[2 * i], v[2 * i + 1]);
    bf[2 * i] = bf_lo(pk);
    bf[2 * i + 1] = bf_hi(pk);
  }
  uint32_t lo = e4m3x2_hw<false>(bf[0], bf[1], 0u);
  lo = e4m3x2_hw<true>(bf[2], bf[3], lo);
  uint32_t hi = e4m3x2_hw<false>(bf[4], bf[5], 0u);
  hi = e4m3x2_hw<true>(bf[6], bf[7], hi);
  return make_uint2(lo, hi);
}

// Keeps the compiler from starting the arithmetic on a QPrep8In before this
// point (it would wait for the loads there, ahead of later loads).
__device__ inline void qprep8_fence(QPrep8In& in) {
  asm volatile("" : "+v"(in.q.x), "+v"(in.q.y), "+v"(in.q.z), "+v"(in.q.w));
  asm volatile("" : "+v"(in.c.x), "+v"(in.c.y), "+v"(in.c.z), "+v"(in.c.w));
  asm volatile("" : "+v"(in.s.x), "+v"(in.s.y), "+v"(in.s.z), "+v"(in.s.w));
  asm volatile("" : "+v"(in.w0.x), "+v"(in.w0.y), "+v"(in.w0.z), "+v"(in.w0.w));
  asm volatile("" : "+v"(in.w1.x), "+v"(in.w1.y), "+v"(in.w1.z), "+v"(in.w1.w));
}

__device__ inline int64_t qprep_pos(int64_t p, int64_t rope_rows) {
  return (p < 0 || p >= rope_rows) ? 0 : p;  // such a row selects nothing later; keep reads in range
}

__device__ inline uint2 qprep8(int mode, const void* __restrict__ qin, int64_t qs, int64_t r,
                               int h, int c, int lane, const float* __restrict__ w, float eps,
                               const uint16_t* __restrict__ rope, int64_t rope_rows,
                               const int64_t* __restrict__ row_pos) {
  if (mode == 1)
    return *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(qin) + r * qs + h * 64 + c * 8);
  const QPrep8In in = qprep8_load(static_cast<const uint16_t*>(qin), qs, r, h, c, w, rope,
                                  qprep_pos(row_pos[r], rope_rows));
  return qprep8_math(in, c, lane, eps);
}

// q prep kernel: one 8-lane group per (row, head)
__global__ __launch_bounds__(256) void qprep_kernel(int mode, const void* __restrict__ qin,
                                                    int64_t qs, int32_t rows,
                                                    const float* __restrict__ w, float eps,
                                                    const uint16_t* __restrict__ rope,
                                                    int64_t rope_rows,
                                                    const int64_t* __restrict__ row_pos,
                                                    uint8_t* __restrict__ q8,
                                                    unsigned* __restrict__ arrivals) {
  const int lane = threadIdx.x & 63;
  const int c = threadIdx.x & 7;
  const int64_t vec = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  {
    // the selection pass of this call counts chunk arrivals per (row, group)
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u < (int64_t)rows * 4) arrivals[u] = 0u;
  }
  if (vec >= (int64_t)rows * 16) return;  // whole 8-lane groups leave together
  const int64_t r = vec >> 4;
  const int h = (int)(vec & 15);
  const uint2 pk = qprep8(mode, qin, qs, r, h, c, lane, w, eps, rope, rope_rows, row_pos);
  *reinterpret_cast<uint2*>(q8 + vec * 64 + c * 8) = pk;
}

hipError_t launch_qprep(const QPrepArgs& a, hipStream_t stream) {
  const int64_t vecs = (int64_t)a.rows * 16;
  if (vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)((vecs + 31) / 32)), dim3(256), 0, stream,
                     a.prepared ? 1 : 0, a.q, a.q_stride_row, a.rows, a.w, a.eps,
                     (const uint16_t*)a.rope, a.rope_rows, a.row_pos, a.q8, a.arrivals);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// score intervals
// ---------------------------------------------------------------------------
constexpr int SC_CB = 64;  // candidates per block (decode: one per wave-row; prefill: 16 per wave)

__global__ __launch_bounds__(256) void score_kernel(
    const uint8_t* __restrict__ q8, int64_t qs8, int32_t rows, const float* __restrict__ w_head,
    int64_t w_stride, const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos,
    const uint8_t* __restrict__ S, int64_t B, int64_t R_cap, int64_t ssb, int64_t pos_limit,
    float2* __restrict__ bounds) {
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
  int32_t s0 = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (seq[i] >= 0) {
      if (s0 < 0) s0 = seq[i];
      else if (seq[i] != s0) shared = false;
    }
  }
  // rows of different sequences: wave w scores row r0 + w over candidates
  // cb0..jend-1; its 64 candidates' loads (16 per lane) are issued first.
  // In iteration u, column n of
  // the MFMA's B operand is candidate cb0 + 4u + n/4 of group
  // ((n & 3) + u) & 3 (the 1 KB of four candidates, the groups rotated by u)
  const bool dec_live = !shared && wave < nr && seq[wave] >= 0 && cb0 < ncand[wave];
  const int64_t jend = dec_live ? ((cb0 + SC_CB < ncand[wave]) ? cb0 + SC_CB : ncand[wave]) : 0;
  uint4 bq[SC_CB / 4];
  if (dec_live) {
    const uint8_t* Sb = S + (int64_t)seq[wave] * ssb;
#pragma unroll
    for (int u = 0; u < SC_CB / 4; ++u) {
      // candidates past jend load candidate jend - 1 again (not stored)
      const int64_t j = cb0 + u * 4 + (n >> 2);
      const int64_t jl = j < jend ? j : jend - 1;
      bq[u] = ldg16(Sb + jl * 256 + (((n & 3) + u) & 3) * 64 + 16 * qd);
    }
  }
  if (cb0 >= maxc) return;

  if (shared) {
    // ---- one sequence: A = (4 rows x 4 heads of group g), B = 16 candidates of g
    const uint8_t* Sb = S + (int64_t)s0 * ssb;
    const int rr = n >> 2, hh = n & 3;
    Bf16x16 aq[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (rr < nr && seq[rr] >= 0)
        raw = ldg16(q8 + (int64_t)(r0 + rr) * qs8 + (4 * g + hh) * 64 + 16 * qd);
      aq[g] = widen16(raw);
    }
    const int orow = r0 + qd;
    const bool orow_ok = qd < nr && seq[qd] >= 0;
    const int64_t onc = orow_ok ? ncand[qd] : 0;
    float w4[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[g][i] = orow_ok ? w_head[(int64_t)orow * w_stride + 4 * g + i] : 0.f;

    const int64_t j = cb0 + wave * 16 + n;  // this lane's candidate column
    uint4 bq[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      bq[g] = (j < maxc) ? ldg16(Sb + j * 256 + g * 64 + 16 * qd) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 d, a;
      dot64(aq[g], widen16(bq[g]), d, a);
      if (j < onc) bounds[((int64_t)orow * 4 + g) * R_cap + j] = score_interval(d, a, w4[g]);
    }
  } else {
    // ---- rows of different sequences (loads issued above)
    if (!dec_live) return;
    const int row = r0 + wave;
    const Bf16x16 aq = widen16(ldg16(q8 + (int64_t)row * qs8 + n * 64 + 16 * qd));
    float w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w4[i] = w_head[(int64_t)row * w_stride + 4 * qd + i];
    // output lane (n, qd) holds heads 4qd..4qd+3 of column n: the result is
    // one of the row's (group qd) in the iteration u with ((n & 3) + u) & 3
    // == qd, once in every four; those are kept and scored four at a time
    const int mu = (qd - (n & 3)) & 3;
    f32x4 dk = {0.f, 0.f, 0.f, 0.f}, ak = dk;
#pragma unroll
    for (int u = 0; u < SC_CB / 4; ++u) {
      f32x4 d, a;
      dot64(aq, widen16(bq[u]), d, a);
      const bool mine = (u & 3) == mu;
      dk = mine ? d : dk;
      ak = mine ? a : ak;
      if ((u & 3) == 3) {
        const int64_t j = cb0 + (u - 3 + mu) * 4 + (n >> 2);
        const float2 iv = score_interval(dk, ak, w4);
        if (j < jend) bounds[((int64_t)row * 4 + qd) * R_cap + j] = iv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// exact scores on the fp64 matrix cores (few rows): one block per (row, 256
// candidates), wave w scoring candidates cb0 + 64w .. cb0 + 64w + 63 in 16
// quads. v_mfma_f64_4x4x4f64 runs 4 independent 4x4x4 blocks; block b is KV
// group g = b, with A[i][k] = the query of head 4g + i and B[k][j] = the
// summary of candidate j of the quad, group g. Lane 16k + 4g + i holds A and
// lane 16k + 4g + j holds B; step t of 16 covers dims 16k + t, so each lane
// loads its 16 contiguous summary bytes (dims 16k..16k+15 of one candidate
// and group) and its 16 query values once. D[i][j] lands in lane
// 16i + 4g + j. All products are exact in fp64, and so is every partial sum
// (a multiple of 2^-18 below 2^24), so the dots are exact in any order; the
// score is then rounded as the oracle rounds it (exact.hpp). Waves 0 and 1
// prep the row's 16 heads into LDS once per block (the same steps as
// qprep_kernel); the first candidate block zeroes the row's top-k arrival
// counters. The prep's loads are issued first, then each wave's first 8
// quads of summary loads, then the prep's arithmetic. With `pool` (units cut
// into several selection chunks) the block also leaves, per group, 8 keys
// for the selection's threshold: each the best score key among 32 of its
// candidates (candidates j and j ^ 1 of a wave's 16 quads), 0 where none.
// ---------------------------------------------------------------------------
// NQ quads of 4 candidates per wave: 16 (256 candidates per block), or 8
// (128) when a batch has too few rows for 1,024 blocks of 256; POOL: `pool`
// is given (the threshold keys are written)
template <bool PREPARED, int NQ, bool POOL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void score_exact_mfma_kernel(
    const float* __restrict__ w_head, int64_t w_stride, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, const uint8_t* __restrict__ S, int64_t B, int64_t R_cap,
    int64_t ssb, int64_t pos_limit, float* __restrict__ scores, uint32_t* __restrict__ pool,
    QPrepArgs prep) {
  __shared__ __align__(16) uint8_t q_lds[16 * 64];
  constexpr int CW = 4 * NQ, CB = 4 * CW;  // candidates per wave, per block
  __shared__ uint32_t pmax[4][8];  // pool: the best key of each 32 candidates (see below)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (threadIdx.x < 32) pmax[threadIdx.x >> 3][threadIdx.x & 7] = 0u;
  const int k = lane >> 4, g = (lane >> 2) & 3, ij = lane & 3;  // ij: head i (A) or candidate j (B)
  const int64_t row = blockIdx.y;
  const int32_t s = row_seq[row];
  const int64_t p = row_pos[row];
  const bool ok = s >= 0 && s < B && p >= 0 && p < pos_limit && (p >> 3) <= R_cap;
  const int64_t nc = ok ? (p >> 3) : 0;
  if (blockIdx.x == 0 && threadIdx.x < 4) {
    // the selection's arrival counters and (pool selection) survivor counts
    prep.arrivals[row * 4 + threadIdx.x] = 0u;
    prep.arrivals[(int64_t)prep.rows * 4 + row * 4 + threadIdx.x] = 0u;
  }
  if ((int64_t)blockIdx.x * CB >= nc) return;  // block-uniform
  const int64_t cb0 = (int64_t)blockIdx.x * CB + CW * wave;
  const bool live = cb0 < nc;
  const int64_t jend = live ? (cb0 + CW < nc ? cb0 + CW : nc) : 0;
  // The query prep's loads go out first (every wave loads the heads of wave
  // & 1, waves 0 and 1 store the result), then the summary loads, so that
  // the prep waits for its own loads only.
  const int ph = 8 * (wave & 1) + (lane >> 3), pc = lane & 7;
  QPrep8In pin;
  uint2 pre;
  if constexpr (PREPARED)
    pre = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(prep.q) +
                                          row * prep.q_stride_row + ph * 64 + pc * 8);
  else
    pin = qprep8_load(static_cast<const uint16_t*>(prep.q), prep.q_stride_row, row, ph, pc,
                      prep.w, static_cast<const uint16_t*>(prep.rope), qprep_pos(p, prep.rope_rows));
  // this lane's 16 summary bytes of quad u: candidate cb0 + 4u + ij, group
  // g, dims 16k..16k+15, through a buffer resource over exactly the wave's
  // jend - cb0 summaries: loads of candidates past jend return zeros (not
  // stored; a wave past the row's candidates has none and stops after the
  // prep). Quads are loaded four at a time, two groups ahead of the one
  // computed.
  const uint8_t* Sw = S + (int64_t)s * ssb + (live ? cb0 * 256 : 0);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Sw, (short)0, (int)(live ? (uint32_t)(jend - cb0) * 256u : 0u), RAW_RSRC3);
  const uint32_t lo = (uint32_t)(ij * 256 + g * 64 + 16 * k);
  auto load4 = [&](int u0, uint4 (&dst)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dst[q] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(lo + 1024u * (u0 + q)), 0, 0));
  };
  uint4 bA[4], bB[4], bC[4];
  load4(0, bA);
  load4(4, bB);
  uint2 pk;
  if constexpr (PREPARED) {
    pk = pre;
  } else {
    qprep8_fence(pin);
    pk = qprep8_math(pin, pc, lane, prep.eps);
  }
  if (wave < 2) *reinterpret_cast<uint2*>(&q_lds[ph * 64 + pc * 8]) = pk;
  __syncthreads();
  // pool: per (row, group), one key per 32 candidates, the best (0 if none),
  // gathered by LDS atomic max. NQ = 16: entry 8 b + 2 wave + p from the
  // lanes of candidates 2p and 2p + 1 of group g (pmax[wave][2g + p]);
  // NQ = 8: entry 4 b + wave from all of the group's lanes (pmax[wave][g]).
  // A unit's keys start every 8 * ceil(R_cap / 256) entries.
  constexpr int PSH = NQ == 16 ? 1 : 2;  // (lane & 15) >> PSH: the lane's pmax slot
  auto pool_put = [&]() {
    const int64_t ustride = ((R_cap + 255) >> 8) * 8;
    if (NQ == 16 && lane < 8)
      pool[(row * 4 + (lane >> 1)) * ustride + 8 * (int64_t)blockIdx.x + 2 * wave + (lane & 1)] =
          pmax[wave][lane];
    if (NQ == 8 && lane < 4)
      pool[(row * 4 + lane) * ustride + 4 * (int64_t)blockIdx.x + wave] = pmax[wave][lane];
  };
  if (!live) {
    if (POOL) pool_put();
    return;
  }
  // A operand: head 4g + ij, dims 16k..16k+15 as packed e4m3, converted per use
  const uint4 qraw = *reinterpret_cast<const uint4*>(&q_lds[(4 * g + ij) * 64 + 16 * k]);
  const uint32_t qw[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
  // this lane's weight for the epilogue: head 4g + i with i = lane >> 4 (the D row)
  const float wl = w_head[row * w_stride + 4 * g + (lane >> 4)];
  // the row's 4 x R_cap scores as one buffer resource; lane offset of its
  // group's candidate cb0
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scores + row * 4 * R_cap), (short)0, (int)(16 * R_cap), RAW_RSRC3);
  const uint32_t obase = (uint32_t)((g * R_cap + cb0) * 4);
  const uint32_t nw = (uint32_t)(jend - cb0);
  auto quads4 = [&](int u0, const uint4 (&bq)[4]) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int m = 0; m < 4; ++m) {  // dword m of the 16 bytes: steps 4m .. 4m+3
      const f32x2 ql = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw[m], false);
      const f32x2 qh = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw[m], true);
      const double qa[4] = {(double)ql[0], (double)ql[1], (double)qh[0], (double)qh[1]};
      double sv[4][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 r4 = bq[q];
        const uint32_t wd = m == 0 ? r4.x : m == 1 ? r4.y : m == 2 ? r4.z : r4.w;
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd, true);
        sv[q][0] = (double)lo[0];
        sv[q][1] = (double)lo[1];
        sv[q][2] = (double)hi[0];
        sv[q][3] = (double)hi[1];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[q] = __builtin_amdgcn_mfma_f64_4x4x4f64(qa[e], sv[q][e], acc[q], 0, 0, 0);
    }
    // D lane 16i + 4g + j: dot of head 4g + i with candidate j of quad q.
    // Each lane weighs its relu term, then a 4 x 4 transpose over (lane row
    // i, quad q), two 32-lane and two 16-lane swaps, leaves in lane
    // 16r + 4g + j the four heads' terms of quad r's candidate j, which it
    // sums in head order.
    uint32_t t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = __float_as_uint(relu0((float)acc[q]) * wl);
    transpose_rows4(t);  // t[i] in lane 16r + 4g + j: head i, quad r
    float sc = __uint_as_float(t[0]) + __uint_as_float(t[1]);
    sc = sc + __uint_as_float(t[2]);
    sc = sc + __uint_as_float(t[3]);
    // candidate cb0 + jw; lanes past jend store to an offset beyond the
    // resource's records (dropped) and put a 0 key, so no lane branches
    const uint32_t jw = (uint32_t)(4 * (u0 + k) + ij);
    const bool in = jw < nw;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), ro,
                                          (int)(in ? obase + 4u * jw : RAW_PAST_END), 0, 0);
    if (POOL) atomicMax(&pmax[wave][(lane & 15) >> PSH], in ? ord_key(sc) : 0u);
  };
  if constexpr (NQ == 16) {
    load4(8, bC);
    quads4(0, bA);
    load4(12, bA);
    quads4(4, bB);
    quads4(8, bC);
    quads4(12, bA);
  } else {
    quads4(0, bA);
    quads4(4, bB);
  }
  if (POOL) pool_put();  // the wave's own LDS atomics precede its reads
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.rows == 0 || a.R_cap == 0) return hipSuccess;
  if (a.exact) {
    // half-size blocks when 256-candidate blocks would not reach 1,024
    const bool half = (int64_t)a.rows * ((a.R_cap + 255) / 256) < 1024;
    const int64_t cb = half ? 128 : 256;
    const dim3 grid((unsigned)((a.R_cap + cb - 1) / cb), (unsigned)a.rows);
    float* const sc = reinterpret_cast<float*>(a.bounds);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, a.w_head, a.w_stride_row, a.row_seq,
                         a.row_pos, a.summary, a.B, a.R_cap, a.ssb, a.pos_limit, sc, a.pool,
                         a.prep);
    };
    const bool pl = a.pool != nullptr;
    if (a.prep.prepared) {
      if (half) pl ? go(score_exact_mfma_kernel<true, 8, true>) : go(score_exact_mfma_kernel<true, 8, false>);
      else pl ? go(score_exact_mfma_kernel<true, 16, true>) : go(score_exact_mfma_kernel<true, 16, false>);
    } else {
      if (half) pl ? go(score_exact_mfma_kernel<false, 8, true>) : go(score_exact_mfma_kernel<false, 8, false>);
      else pl ? go(score_exact_mfma_kernel<false, 16, true>) : go(score_exact_mfma_kernel<false, 16, false>);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.R_cap + SC_CB - 1) / SC_CB), (unsigned)((a.rows + 3) / 4));
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, stream, a.q8, a.q8_stride_row, a.rows,
                     a.w_head, a.w_stride_row, a.row_seq, a.row_pos, a.summary, a.B, a.R_cap,
                     a.ssb, a.pos_limit, a.bounds);
  return hipGetLastError();
}

}  // namespace s5
