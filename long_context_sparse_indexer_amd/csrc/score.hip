// Indexer query prep and region scoring.
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// the indexer q has 16 heads, RMSNorm with scale (1 + w) and NEOX rotation of
// dims 0..31; a region's score for a KV group is the sum over the group's
// heads of relu(e4m3(q_h) . summary) * w_h; the top 512 by (-score, id) are
// kept in that order.
//
// q prep rounding points (fp32): ms = sum64(x*x)/64, r = 1/sqrt(ms + eps),
// y = (x*r)*(1 + w), rotation a*c - b*s | b*c + a*s from bf16 cos/sin, bf16,
// then e4m3.
//
// Exact dot products. Every e4m3 x e4m3 product has at most 8 significant
// bits, and any partial sum of 64 of them is a multiple of 2^-18 below 2^24
// in magnitude (at most 42 significant bits), so fp64 fused multiply-adds
// accumulate the dot product with no rounding at all, in any order. The one
// rounding is the final fp64 -> fp32, which makes every score the exact
// value rounded once: identical to any other exact implementation, so the
// (-score, id) order and therefore the selected ids are reproducible bit for
// bit. (fp8 matrix cores accumulate in fp32 and reorder candidates whose
// scores differ by a few fp32 ulps, which is common among 10^4..10^5
// candidates.)
//
// Mapping: q prep writes the e4m3 query as exact fp64 values laid out
// [row][group][dim][4 heads], so that a wave reads its group's query through
// scalar loads. In the score kernel wave w of a block handles group w and
// lane l one candidate: the lane reads the candidate's 64-byte group vector
// (four 16-byte loads), converts it to fp64 once, and reuses it for every
// row of the block's row tile that reads the same sequence (a prefill chunk
// shares it across the tile; decode rows each bring their own).
// Epilogue per (row, group, candidate): t_h = max(fp32(dot_h), +0), then
// ((t0*w0 + t1*w1) + t2*w2) + t3*w3 with separately rounded products.
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

// exact value of an e4m3 code (finite codes)
__device__ inline double e4m3_f64(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  double v;
  if (e == 0) {
    v = (double)m * 0x1p-9;
  } else {
    const unsigned long long bits = ((unsigned long long)(e + 1016u) << 52) | ((unsigned long long)m << 49);
    v = __builtin_bit_cast(double, bits);
  }
  return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------------------
// q prep: one 8-lane group per (row, head); lane c holds dims 8c..8c+7.
// mode 0: bf16 input, full prep; mode 1: the input is already e4m3.
// Writes q64[row][h/4][dim][h%4] (fp64 values of the e4m3 codes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qprep_kernel(int mode, const void* __restrict__ qin,
                                                    int64_t qs, int32_t rows,
                                                    const float* __restrict__ w, float eps,
                                                    const uint16_t* __restrict__ rope,
                                                    int64_t rope_rows,
                                                    const int64_t* __restrict__ row_pos,
                                                    double* __restrict__ q64) {
  const int lane = threadIdx.x & 63;
  const int c = threadIdx.x & 7;
  const int64_t vec = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  if (vec >= (int64_t)rows * 16) return;  // whole 8-lane groups leave together
  const int64_t r = vec >> 4;
  const int h = (int)(vec & 15);
  uint32_t code[8];
  if (mode == 1) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(qin) + r * qs + h * 64 + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      code[i] = (raw.x >> (8 * i)) & 0xffu;
      code[4 + i] = (raw.y >> (8 * i)) & 0xffu;
    }
  } else {
    const uint16_t* q = static_cast<const uint16_t*>(qin);
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
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float other = dpp<DPP_QUAD_XOR2>(y[i]);
      const float own_c = y[i] * cf[i];
      const float oth_s = other * sf[i];
      const float rot = first_half ? (own_c - oth_s) : (own_c + oth_s);
      code[i] = e4m3_from_bf16(bf16_bits(rotated ? rot : y[i]));
    }
  }
  double* dst = q64 + ((r * 4 + (h >> 2)) * 64 + c * 8) * 4 + (h & 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i * 4] = e4m3_f64(code[i]);
}

hipError_t launch_qprep(const QPrepArgs& a, hipStream_t stream) {
  const int64_t vecs = (int64_t)a.rows * 16;
  if (vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)((vecs + 31) / 32)), dim3(256), 0, stream,
                     a.prepared ? 1 : 0, a.q, a.q_stride_row, a.rows, a.w, a.eps,
                     (const uint16_t*)a.rope, a.rope_rows, a.row_pos, a.q64);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------
constexpr int SC_RT = 8;   // rows per tile
constexpr int SC_CB = 64;  // candidates per block (one per lane)

__device__ inline float relu0(float v) { return v > 0.0f ? v : 0.0f; }

__global__ __launch_bounds__(256) void score_kernel(
    const double* __restrict__ q64, int32_t rows, const float* __restrict__ w_head,
    int64_t w_stride, const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos,
    const uint8_t* __restrict__ S, int64_t B, int64_t R_cap, int64_t ssb, int64_t pos_limit,
    float* __restrict__ scores) {
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the wave's group
  const int lane = threadIdx.x & 63;
  const int r0 = blockIdx.y * SC_RT;
  const int64_t j = (int64_t)blockIdx.x * SC_CB + lane;
  const int nr = min(SC_RT, rows - r0);

  int32_t seq[SC_RT];
  int64_t ncand[SC_RT];
  int64_t maxc = 0;
#pragma unroll
  for (int i = 0; i < SC_RT; ++i) {
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
  if ((int64_t)blockIdx.x * SC_CB >= maxc) return;

  uint32_t done = 0;
  for (int i = 0; i < nr; ++i) {
    if (seq[i] < 0 || ((done >> i) & 1u)) continue;
    const int32_t s = seq[i];
    int64_t nc_s = 0;  // candidates any row of this sequence needs
#pragma unroll
    for (int i2 = 0; i2 < SC_RT; ++i2)
      if (seq[i2] == s && ncand[i2] > nc_s) nc_s = ncand[i2];
    // this lane's candidate vector for group g, as exact fp64
    double sv[64];
    if (j < nc_s) {
      const uint8_t* src = S + (int64_t)s * ssb + j * 256 + g * 64;
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        const uint4 raw = ldg16(src + 16 * part);
        const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], true);
          sv[16 * part + 4 * k + 0] = (double)lo.x;
          sv[16 * part + 4 * k + 1] = (double)lo.y;
          sv[16 * part + 4 * k + 2] = (double)hi.x;
          sv[16 * part + 4 * k + 3] = (double)hi.y;
        }
      }
    } else {
#pragma unroll
      for (int d = 0; d < 64; ++d) sv[d] = 0.0;
    }
    for (int i2 = i; i2 < nr; ++i2) {
      if (seq[i2] != s) continue;
      done |= 1u << i2;
      const int row = r0 + i2;
      const double* qg = q64 + ((int64_t)row * 4 + g) * 256;  // [64 dims][4 heads], wave-uniform
      double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
      for (int d = 0; d < 64; ++d) {
        a0 = fma(qg[4 * d + 0], sv[d], a0);
        a1 = fma(qg[4 * d + 1], sv[d], a1);
        a2 = fma(qg[4 * d + 2], sv[d], a2);
        a3 = fma(qg[4 * d + 3], sv[d], a3);
      }
      if (j < ncand[i2]) {
        const float* w4 = w_head + (int64_t)row * w_stride + 4 * g;
        const float t0 = relu0((float)a0) * w4[0];
        const float t1 = relu0((float)a1) * w4[1];
        const float t2 = relu0((float)a2) * w4[2];
        const float t3 = relu0((float)a3) * w4[3];
        float sc = t0 + t1;
        sc = sc + t2;
        sc = sc + t3;
        scores[((int64_t)row * 4 + g) * R_cap + j] = sc;
      }
    }
  }
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.rows == 0 || a.R_cap == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.R_cap + SC_CB - 1) / SC_CB), (unsigned)((a.rows + SC_RT - 1) / SC_RT));
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, stream, a.q64, a.rows, a.w_head,
                     a.w_stride_row, a.row_seq, a.row_pos, a.summary, a.B, a.R_cap, a.ssb,
                     a.pos_limit, a.scores);
  return hipGetLastError();
}

}  // namespace s5
