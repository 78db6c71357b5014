// Score intervals on the bf16 matrix cores, shared by the interval scorer
// and the fused prefill selection.
//
// Every e4m3 value is exactly a bf16 value, so a 64-dim e4m3 dot runs as two
// 16x16x32 bf16 MFMAs with fp32 accumulation; the same MFMAs on absolute
// values give A = sum |q s|. Accumulation may round, so the score of a
// candidate is returned as an interval that holds the exact score (bound
// derived and measured in score.hip's header).
#pragma once

#include "device.hpp"
#include "exact.hpp"

namespace s5 {

// 16 e4m3 bytes -> 16 bf16 (two 8-element MFMA operands), exactly
struct Bf16x16 {
  uint4 lo, hi;
};
// bytes 2*UPPER, 2*UPPER + 1 of w as two bf16 (the first in the low half):
// gfx950's scaled fp8 -> bf16 conversion with scale 1, exact since every
// e4m3 value is a bf16 value
template <bool UPPER>
__device__ inline uint32_t widen2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, UPPER));
}
__device__ inline Bf16x16 widen16(uint4 v) {
  Bf16x16 r;
  r.lo = make_uint4(widen2<false>(v.x), widen2<true>(v.x), widen2<false>(v.y), widen2<true>(v.y));
  r.hi = make_uint4(widen2<false>(v.z), widen2<true>(v.z), widen2<false>(v.w), widen2<true>(v.w));
  return r;
}
__device__ inline uint4 abs_bf16(uint4 v) {
  return make_uint4(v.x & 0x7fff7fffu, v.y & 0x7fff7fffu, v.z & 0x7fff7fffu, v.w & 0x7fff7fffu);
}
__device__ inline f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// dot over the 64 dims and the same over absolute values
__device__ inline void dot64(const Bf16x16& a, const Bf16x16& b, f32x4& d, f32x4& ad) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  d = mfma_bf16(a.hi, b.hi, mfma_bf16(a.lo, b.lo, z));
  ad = mfma_bf16(abs_bf16(a.hi), abs_bf16(b.hi), mfma_bf16(abs_bf16(a.lo), abs_bf16(b.lo), z));
}

// interval [lo, hi] around the approximate score of one (row, group, candidate)
__device__ inline float2 score_interval(f32x4 d, f32x4 a, const float* w4) {
  const float s = group_score4(d[0], d[1], d[2], d[3], w4);
  const float aw = fabsf(w4[0]) * a[0] + fabsf(w4[1]) * a[1] + fabsf(w4[2]) * a[2] +
                   fabsf(w4[3]) * a[3];
  const float delta = 0x1p-18f * aw + 0x1p-22f * fabsf(s);
  return make_float2(s - delta, s + delta);
}

}  // namespace s5
