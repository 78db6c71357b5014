// Exact region scores: the arithmetic shared by the scoring and selection
// kernels.
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

}  // namespace s5
