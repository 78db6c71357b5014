// Shared by summarize.hip and topk.hip: the summary of one region by 256
// lanes, and the append of one decode row's token (its ring slot, and the
// summary of the region the token completes).
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"): the indexer commit
// note summarises every completed 8-token region per dim as a softmax over
// the region's z weighting the prepared k, through bf16 to e4m3; the
// prompt-path commit note keeps the indexer's k and z in rings.
#pragma once

#include "device.hpp"
#include "launch.hpp"

namespace s5 {

// One region by one 256-thread workgroup, lane (t, g, c) = token t, group g,
// dims 8c..8c+7, so the 8 tokens run side by side. The same arithmetic in the
// same order as summarize_kernel: the max over tokens (order-free), each
// token's k prep and e_t, e_t * k_t, then den and num summed in token order by
// the lanes of token 0, from LDS. kt, zt: this lane's 8 dims of its token;
// cs: its token's rope row; dst: the region's 8 output bytes of this lane
// (written by the lanes of token 0). tid: the lane's index among the 256;
// z_lds [8][32] (z, 8 bf16 per token and lane) and ep_lds [8][32][4] (e and
// e*k) in LDS. Contains two workgroup barriers: every thread of the
// workgroup takes part in them (threads past the 256, as whole waves, by two
// barriers of their own).
__device__ inline void summarize_region_lanes(const uint16_t* __restrict__ kt,
                                              const uint16_t* __restrict__ zt,
                                              const uint16_t* __restrict__ cs,
                                              const float* __restrict__ lnw,
                                              const float* __restrict__ lnb, float eps,
                                              uint8_t* __restrict__ dst, int tid,
                                              uint4 (*z_lds)[32], float4 (*ep_lds)[32][4]) {
  const int lane = tid & 63;
  const int t = tid >> 5, sub = tid & 31;
  const int c = sub & 7;
  const uint4 zraw = ldg16(zt);
  const uint4 kraw = ldg16(kt);
  z_lds[t][sub] = zraw;
  float gw[8], gb[8];
  {
    const float4 w0 = reinterpret_cast<const float4*>(lnw)[2 * c];
    const float4 w1 = reinterpret_cast<const float4*>(lnw)[2 * c + 1];
    const float4 b0 = reinterpret_cast<const float4*>(lnb)[2 * c];
    const float4 b1 = reinterpret_cast<const float4*>(lnb)[2 * c + 1];
    gw[0] = w0.x; gw[1] = w0.y; gw[2] = w0.z; gw[3] = w0.w;
    gw[4] = w1.x; gw[5] = w1.y; gw[6] = w1.z; gw[7] = w1.w;
    gb[0] = b0.x; gb[1] = b0.y; gb[2] = b0.z; gb[3] = b0.w;
    gb[4] = b1.x; gb[5] = b1.y; gb[6] = b1.z; gb[7] = b1.w;
  }
  const bool rotated = c < 4;
  const bool first_half = c < 2;
  const int fi = (c & 1) * 8;
  const uint32_t sflip = first_half ? 0x80000000u : 0u;

  // k prep of this lane's token
  float x[8], d[8], d2[8], y[8];
  unpack_bf16x8(kraw, x);
  const float mu = sum8_lanes(pair8(x), lane) / 64.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    d[i] = x[i] - mu;
    d2[i] = d[i] * d[i];
  }
  const float var = sum8_lanes(pair8(d2), lane) / 64.0f;
  const float r = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float tt = (d[i] * r) * gw[i];
    y[i] = tt + gb[i];
  }
  float cf[8], sf[8];
  unpack_bf16x8(ldg16(cs + fi), cf);
  unpack_bf16x8(ldg16(cs + 16 + fi), sf);
  float rv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sfs = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, sf[i]) ^ sflip);
    const float own_c = y[i] * cf[i];
    const float oth_s = dpp<DPP_QUAD_XOR2>(y[i]) * sfs;
    const float rot = own_c + oth_s;
    rv[i] = rotated ? rot : y[i];
  }
  float kv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t pk = bf16x2_hw(rv[2 * i], rv[2 * i + 1]);
    kv[2 * i] = bf_lo(pk);
    kv[2 * i + 1] = bf_hi(pk);
  }
  __syncthreads();
  // the max of each dim over the region's tokens
  float m[8], zf[8];
  unpack_bf16x8(z_lds[0][sub], m);
#pragma unroll
  for (int s2 = 1; s2 < 8; ++s2) {
    unpack_bf16x8(z_lds[s2][sub], zf);
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], zf[i]);
  }
  unpack_bf16x8(zraw, zf);
  float e[8], pr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    e[i] = exp_fixed(zf[i] - m[i]);
    pr[i] = e[i] * kv[i];
  }
  ep_lds[t][sub][0] = make_float4(e[0], e[1], e[2], e[3]);
  ep_lds[t][sub][1] = make_float4(e[4], e[5], e[6], e[7]);
  ep_lds[t][sub][2] = make_float4(pr[0], pr[1], pr[2], pr[3]);
  ep_lds[t][sub][3] = make_float4(pr[4], pr[5], pr[6], pr[7]);
  __syncthreads();
  if (t != 0) return;
  float den[8], num[8];
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) {
    const float4 e0 = ep_lds[s2][sub][0], e1 = ep_lds[s2][sub][1];
    const float4 p0 = ep_lds[s2][sub][2], p1 = ep_lds[s2][sub][3];
    const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
    const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s2 == 0) {
        den[i] = ev[i];
        num[i] = pv[i];
      } else {
        den[i] = den[i] + ev[i];
        num[i] = num[i] + pv[i];
      }
    }
  }
  float sbv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t pk = bf16x2_hw(num[2 * i] / den[2 * i], num[2 * i + 1] / den[2 * i + 1]);
    sbv[2 * i] = bf_lo(pk);
    sbv[2 * i + 1] = bf_hi(pk);
  }
  uint32_t lo = e4m3x2_hw<false>(sbv[0], sbv[1], 0u);
  lo = e4m3x2_hw<true>(sbv[2], sbv[3], lo);
  uint32_t hi = e4m3x2_hw<false>(sbv[4], sbv[5], 0u);
  hi = e4m3x2_hw<true>(sbv[6], sbv[7], hi);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
}


__device__ inline bool append_row_ok(int32_t s, int64_t p, int64_t B, int64_t rope_rows,
                                     int64_t R_cap) {
  return s >= 0 && s < B && p >= 0 && p < rope_rows && (p >> 3) < R_cap;
}

// The append of row r by the first 256 threads of the calling workgroup,
// for calls whose rows are of distinct sequences: the token goes to ring
// slot p mod slots of its sequence, and if it ends a region, the region is
// summarised from the ring's 7 earlier tokens (written by earlier calls; no
// other row of the call writes this sequence's ring) and the token itself,
// read from k_new/z_new. Every thread of the workgroup must call it: the
// early exits are workgroup-uniform, and threads 256 and up (whole waves)
// take part only in the summary's two barriers.
__device__ inline void append_row_block(const AppendArgs& ap, int64_t r, uint4 (*z_lds)[32],
                                        float4 (*ep_lds)[32][4]) {
  const uint16_t* k_new = static_cast<const uint16_t*>(ap.k_new);
  const uint16_t* z_new = static_cast<const uint16_t*>(ap.z_new);
  uint16_t* k_ring = static_cast<uint16_t*>(ap.k_ring);
  uint16_t* z_ring = static_cast<uint16_t*>(ap.z_ring);
  const int64_t nsr = ap.new_stride_row, rsb = ap.ring_stride_b, slots = ap.slots;
  const int32_t s = ap.row_seq[r];
  const int64_t p = ap.row_pos[r];
  if (!append_row_ok(s, p, ap.B, ap.rope_rows, ap.R_cap)) return;  // workgroup-uniform
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int64_t e = (int64_t)(tid & 31) * 8;
    const int64_t dst = (int64_t)s * rsb + (p % slots) * 256 + e;
    if (tid < 32) *reinterpret_cast<uint4*>(k_ring + dst) = ldg16(k_new + r * nsr + e);
    else *reinterpret_cast<uint4*>(z_ring + dst) = ldg16(z_new + r * nsr + e);
  }
  if ((p & 7) != 7) return;  // workgroup-uniform
  if (tid >= 256) {  // whole waves
    __syncthreads();
    __syncthreads();
    return;
  }
  const int t = tid >> 5, sub = tid & 31;
  const int g = sub >> 3, c = sub & 7;
  const int64_t a = p - 7;
  const int64_t io = (int64_t)g * 64 + c * 8;
  const uint16_t* kt = t == 7 ? k_new + r * nsr + io : k_ring + (int64_t)s * rsb + ((a % slots) + t) * 256 + io;
  const uint16_t* zt = t == 7 ? z_new + r * nsr + io : z_ring + (int64_t)s * rsb + ((a % slots) + t) * 256 + io;
  summarize_region_lanes(kt, zt, static_cast<const uint16_t*>(ap.rope) + (a + t) * 32, ap.ln_w,
                         ap.ln_b, ap.eps,
                         static_cast<uint8_t*>(ap.summary) + (int64_t)s * ap.ssb + (p >> 3) * 256 + io,
                         tid, z_lds, ep_lds);
}

}  // namespace s5
