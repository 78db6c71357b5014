// Exact region scores, shared by the scoring and selection kernels.
//
// Every e4m3 x e4m3 product has at most 8 significant bits, and every partial
// sum of 64 of them is a multiple of 2^-18 below 2^24 in magnitude (at most 42
// significant bits), so fp64 fused multiply-adds accumulate the 64-dim dot
// product with no rounding at all, in any order. The score of a candidate for
// a KV group is then fp32(dot_h) for the group's 4 heads, relu (-0 -> +0),
// and ((t0*w0 + t1*w1) + t2*w2) + t3*w3 with separately rounded fp32 products
// (TensorFold #903, "Step-5-Preview on one 256 GB Mac", indexer commit note:
// sum over the group's heads of relu(e4m3(q_h) . summary) * w_h).
#pragma once

#include "device.hpp"

namespace s5 {

__device__ inline float relu0(float v) { return v > 0.0f ? v : 0.0f; }

// the score epilogue from four fp32 dot products
__device__ inline float group_score4(float d0, float d1, float d2, float d3, const float* w4) {
  const float t0 = relu0(d0) * w4[0];
  const float t1 = relu0(d1) * w4[1];
  const float t2 = relu0(d2) * w4[2];
  const float t3 = relu0(d3) * w4[3];
  float s = t0 + t1;
  s = s + t2;
  s = s + t3;
  return s;
}

// Exact score of one candidate from the 64 bytes of its group vector (raw,
// already loaded) and the row's query for the group as exact fp64, laid out
// [64 dims][4 heads].
__device__ inline float exact_group_score_raw(const uint4 (&raw)[4], const double* __restrict__ qg,
                                              const float* __restrict__ w4) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
  for (int part = 0; part < 4; ++part) {
    const uint32_t wds[4] = {raw[part].x, raw[part].y, raw[part].z, raw[part].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], true);
      const float v[4] = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * part + 4 * k + e;
        const double s = (double)v[e];
        a0 = fma(qg[4 * d + 0], s, a0);
        a1 = fma(qg[4 * d + 1], s, a1);
        a2 = fma(qg[4 * d + 2], s, a2);
        a3 = fma(qg[4 * d + 3], s, a3);
      }
    }
  }
  return group_score4((float)a0, (float)a1, (float)a2, (float)a3, w4);
}

// The same with the query in global memory, read in chunks of 4 dims (16
// values) that the compiler keeps in scalar registers when qg is the same in
// every lane; the empty asm statements keep each chunk's loads after the
// previous chunk's products, so only a chunk or two is live at a time.
__device__ inline float exact_group_score_sq(const uint4 (&raw)[4], const double* __restrict__ qg,
                                             const float* __restrict__ w4) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
  for (int part = 0; part < 4; ++part) {
    const uint32_t wds[4] = {raw[part].x, raw[part].y, raw[part].z, raw[part].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)::"memory");
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], true);
      const float v[4] = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * part + 4 * k + e;
        const double s = (double)v[e];
        a0 = fma(qg[4 * d + 0], s, a0);
        a1 = fma(qg[4 * d + 1], s, a1);
        a2 = fma(qg[4 * d + 2], s, a2);
        a3 = fma(qg[4 * d + 3], s, a3);
      }
    }
  }
  return group_score4((float)a0, (float)a1, (float)a2, (float)a3, w4);
}

// the same, loading the 64 bytes at sv
__device__ inline float exact_group_score(const uint8_t* __restrict__ sv,
                                          const double* __restrict__ qg,
                                          const float* __restrict__ w4) {
  const uint4 raw[4] = {ldg16(sv), ldg16(sv + 16), ldg16(sv + 32), ldg16(sv + 48)};
  return exact_group_score_raw(raw, qg, w4);
}

// Exact partial dots over 32 dims for the 4 heads: sv = 32 bytes of the
// candidate's group vector, qh = the query's matching 32 dims [32][4 heads].
__device__ inline void exact_half_dots(const uint8_t* __restrict__ sv, const double* qh,
                                       double* a) {
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const uint4 raw = ldg16(sv + 16 * part);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[k], true);
      const float v[4] = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * part + 4 * k + e;
        const double s = (double)v[e];
        a[0] = fma(qh[4 * d + 0], s, a[0]);
        a[1] = fma(qh[4 * d + 1], s, a[1]);
        a[2] = fma(qh[4 * d + 2], s, a[2]);
        a[3] = fma(qh[4 * d + 3], s, a[3]);
      }
    }
  }
}

}  // namespace s5
