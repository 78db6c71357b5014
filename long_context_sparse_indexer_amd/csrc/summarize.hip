// Region summaries of the indexer keys, with the k prep fused into the load.
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// the indexer k is LayerNormed with bias and NEOX-rotated on dims 0..31;
// every completed 8-token region is summarised per dim as a softmax over the
// region's z weighting k, rounded through bf16 to e4m3.
//
// Fixed rounding points (the path's reading of the note):
//   k prep, per (token, group), fp32:  mu = sum64(x)/64, d = x - mu,
//     var = sum64(d*d)/64, r = 1/sqrt(var + eps), y = (d*r)*gamma + beta,
//     rotation a*c - b*s | b*c + a*s with bf16 cos/sin, then bf16;
//     sum64 = halving tree within each run of 8 dims, then over the runs.
//   summary, per (region, group, dim):  m = max_t z_t, e_t = exp_fixed(z_t - m),
//     den and num summed in token order (num of the rounded products e_t*k_t),
//     s = num/den, code = e4m3(bf16(s)).
// The bf16 and e4m3 roundings use gfx950's conversion instructions
// (bf16x2_hw, e4m3x2_hw), which give the same bits as the software forms.
//
// Mapping: a region is 4 KB of k and 4 KB of z (8 tokens x 4 groups x 64
// bf16, contiguous). 32 lanes own it: lane (g, c) holds dims 8c..8c+7 of group
// g for all 8 tokens, so the 64 dims of a (token, group) sit on 8 adjacent
// lanes (reduced with DPP) and the 8 tokens of a dim sit in one lane. A wave
// covers 2 regions, a 256-thread block 8; every load is 16 B per lane and a
// wave's loads cover whole 512-B token rows. The 256 B of e4m3 a region
// produces are stored 8 B per lane, contiguous across the 32 lanes.
#include "device.hpp"
#include "launch.hpp"
#include "region_block.hpp"

namespace s5 {

// out[t] = v of lane 8 (i / 8) + t (t < 4), for the lanes i of every 8-lane
// group (ds_swizzle in its bit-mask mode: and-mask 0x18 keeps the group,
// or-mask t)
template <int T>
__device__ inline void bcast4_of8(float v, float (&out)[4]) {
  out[T] = __builtin_bit_cast(
      float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x18 | (T << 5)));
  if constexpr (T < 3) bcast4_of8<T + 1>(v, out);
}

__global__ __launch_bounds__(256) void summarize_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ z, int64_t nreg, int64_t total,
    int64_t t0, int64_t sb, int64_t st, const float* __restrict__ lnw,
    const float* __restrict__ lnb, float eps, const uint16_t* __restrict__ rope,
    uint8_t* __restrict__ S, int64_t ssb) {
  const int lane = threadIdx.x & 63;
  const int sub = threadIdx.x & 31;
  const int g = sub >> 3, c = sub & 7;
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
  const bool rotated = c < 4;        // dims 0..31
  const bool first_half = c < 2;     // dims 0..15 hold the pair's first element
  const int fi = (c & 1) * 8;        // frequency index of this lane's first dim
  const int64_t j0 = t0 >> 3;
  // the rope rows of the wave's two regions (16 tokens), as fp32: per token
  // cos 0..15 | sin 0..15 | -sin 0..15. Lane (region half, token sub/4,
  // piece sub%4) stages 8 values; a lane reads cos and its signed sin at
  // dims fi..fi+7 (the first half's a*c - b*s is a*c + b*(-s), negation
  // being exact).
  __shared__ float4 rope_lds[4][2][8][12];
  float4 (*const rw)[12] = rope_lds[threadIdx.x >> 6][(threadIdx.x >> 5) & 1];
  const int st_t = sub >> 2, st_p = sub & 3;
  const int rd_c = fi >> 2, rd_s = (first_half ? 8 : 4) + (fi >> 2);

  for (int64_t u = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5); u < total;
       u += (int64_t)gridDim.x * 8) {
    const int64_t b = u / nreg, jr = u - b * nreg;
    const int64_t off = b * sb + jr * 8 * st + g * 64 + c * 8;
    const uint16_t* kp = k + off;
    const uint16_t* zp = z + off;

    uint4 zr[8], kr[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) zr[t] = ldg16(zp + t * st);
#pragma unroll
    for (int t = 0; t < 8; ++t) kr[t] = ldg16(kp + t * st);

    float m[8];
    unpack_bf16x8(zr[0], m);
#pragma unroll
    for (int t = 1; t < 8; ++t) {
      float zt[8];
      unpack_bf16x8(zr[t], zt);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], zt[i]);
    }
    // z stays packed until each token's exponentials (unpacked again there)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __asm__ volatile("" : "+v"(zr[t].x), "+v"(zr[t].y));
      __asm__ volatile("" : "+v"(zr[t].z), "+v"(zr[t].w));
    }

    float den[8], num[8];
    {
      const uint16_t* cs = rope + (t0 + jr * 8) * 32;
      float f[8];
      unpack_bf16x8(ldg16(cs + st_t * 32 + st_p * 8), f);
      const int o = st_p < 2 ? 2 * st_p : 4 + 2 * (st_p - 2);
      rw[st_t][o] = make_float4(f[0], f[1], f[2], f[3]);
      rw[st_t][o + 1] = make_float4(f[4], f[5], f[6], f[7]);
      if (st_p >= 2) {
        rw[st_t][o + 4] = make_float4(-f[0], -f[1], -f[2], -f[3]);
        rw[st_t][o + 5] = make_float4(-f[4], -f[5], -f[6], -f[7]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // the tokens in two halves of four: k prep statistics (mean and variance
    // per (token, group), every lane of the group holding its dims'
    // deviations), then r = 1/sqrt(var + eps) of token 4h + c % 4 once per
    // lane (lane (g, c) of the region's 32), token t's r taken from lane
    // (g, t % 4) of the same 8 lanes, then the rest of the token's work
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float d[4][8], var[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        float x[8], d2[8];
        unpack_bf16x8(kr[4 * h + t4], x);
        const float mu = sum8_lanes(pair8(x), lane) / 64.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          d[t4][i] = x[i] - mu;
          d2[i] = d[t4][i] * d[t4][i];
        }
        var[t4] = sum8_lanes(pair8(d2), lane) / 64.0f;
      }
      const int c4 = c & 3;
      const float vc = c4 < 2 ? (c4 == 0 ? var[0] : var[1]) : (c4 == 2 ? var[2] : var[3]);
      const float rc = 1.0f / sqrtf(vc + eps);
      float rt[4];
      bcast4_of8<0>(rc, rt);
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int t = 4 * h + t4;
        const float r = rt[t4];
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float tt = (d[t4][i] * r) * gw[i];
          y[i] = tt + gb[i];
        }
        // NEOX rotation: lanes c and c^2 (c < 4) hold the two halves of the
        // pairs
        float cf[8], sfs[8];
        {
          // (read here, not hoisted to the loop top: the rows of all eight
          // tokens at once would double the live registers)
          __asm__ volatile("" ::: "memory");
          const float4 c0 = rw[t][rd_c], c1 = rw[t][rd_c + 1];
          const float4 s0 = rw[t][rd_s], s1 = rw[t][rd_s + 1];
          cf[0] = c0.x; cf[1] = c0.y; cf[2] = c0.z; cf[3] = c0.w;
          cf[4] = c1.x; cf[5] = c1.y; cf[6] = c1.z; cf[7] = c1.w;
          sfs[0] = s0.x; sfs[1] = s0.y; sfs[2] = s0.z; sfs[3] = s0.w;
          sfs[4] = s1.x; sfs[5] = s1.y; sfs[6] = s1.z; sfs[7] = s1.w;
        }
        float rv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float own_c = y[i] * cf[i];
          const float oth_s = dpp<DPP_QUAD_XOR2>(y[i]) * sfs[i];
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
        float zf[8];
        unpack_bf16x8(zr[t], zf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = exp_fixed(zf[i] - m[i]);
          const float pr = e * kv[i];
          if (t == 0) {
            den[i] = e;
            num[i] = pr;
          } else {
            den[i] = den[i] + e;
            num[i] = num[i] + pr;
          }
        }
      }
    }
    float sb[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t pk = bf16x2_hw(num[2 * i] / den[2 * i], num[2 * i + 1] / den[2 * i + 1]);
      sb[2 * i] = bf_lo(pk);
      sb[2 * i + 1] = bf_hi(pk);
    }
    uint32_t lo = e4m3x2_hw<false>(sb[0], sb[1], 0u);
    lo = e4m3x2_hw<true>(sb[2], sb[3], lo);
    uint32_t hi = e4m3x2_hw<false>(sb[4], sb[5], 0u);
    hi = e4m3x2_hw<true>(sb[6], sb[7], hi);
    uint2* dst = reinterpret_cast<uint2*>(S + b * ssb + (j0 + jr) * 256 + g * 64 + c * 8);
    *dst = make_uint2(lo, hi);
  }
}

// summarize_region_lanes for a 256-thread workgroup, LDS of its own
__device__ inline void summarize_region_block(const uint16_t* __restrict__ kt,
                                              const uint16_t* __restrict__ zt,
                                              const uint16_t* __restrict__ cs,
                                              const float* __restrict__ lnw,
                                              const float* __restrict__ lnb, float eps,
                                              uint8_t* __restrict__ dst) {
  __shared__ uint4 z_lds[8][32];
  __shared__ float4 ep_lds[8][32][4];
  summarize_region_lanes(kt, zt, cs, lnw, lnb, eps, dst, (int)threadIdx.x, z_lds, ep_lds);
}

// Few regions (a decode step's own regions, a prefill chunk): one workgroup
// per region of the span.
__global__ __launch_bounds__(256) void summarize_small_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ z, int64_t nreg,
    int64_t t0, int64_t sb, int64_t st, const float* __restrict__ lnw,
    const float* __restrict__ lnb, float eps, const uint16_t* __restrict__ rope,
    uint8_t* __restrict__ S, int64_t ssb) {
  const int t = threadIdx.x >> 5, sub = threadIdx.x & 31;
  const int g = sub >> 3, c = sub & 7;
  const int64_t u = blockIdx.x;
  const int64_t b = u / nreg, jr = u - b * nreg;
  const int64_t off = b * sb + (jr * 8 + t) * st + g * 64 + c * 8;
  summarize_region_block(k + off, z + off, rope + (t0 + jr * 8 + t) * 32, lnw, lnb, eps,
                         S + b * ssb + ((t0 >> 3) + jr) * 256 + g * 64 + c * 8);
}

// ---------------------------------------------------------------------------
// Incremental update of the k/z rings (TensorFold #903, prompt-path commit
// note: the indexer keeps its k and z in rings; indexer commit note: every
// completed region is summarised). Step 1 writes every row's token to slot
// p mod slots of its sequence; step 2, a second launch so that it sees every
// token of step 1, summarises the region each row's token completes, from
// the ring (a region's 8 slots are contiguous: slots is a multiple of 8).
// ---------------------------------------------------------------------------
// one wave per row: lanes 0..31 copy the 512 B of k, lanes 32..63 those of z
__global__ __launch_bounds__(256) void append_scatter_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ z_new, int64_t nsr,
    const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos, int32_t rows,
    uint16_t* __restrict__ k_ring, uint16_t* __restrict__ z_ring, int64_t B, int64_t slots,
    int64_t rsb, int64_t rope_rows, int64_t R_cap) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int32_t s = row_seq[r];
  const int64_t p = row_pos[r];
  if (!append_row_ok(s, p, B, rope_rows, R_cap)) return;
  const int lane = threadIdx.x & 63;
  const int64_t e = (int64_t)(lane & 31) * 8;  // this lane's 8 bf16 of the token's 256
  const int64_t dst = (int64_t)s * rsb + (p % slots) * 256 + e;
  if (lane < 32) *reinterpret_cast<uint4*>(k_ring + dst) = ldg16(k_new + r * nsr + e);
  else *reinterpret_cast<uint4*>(z_ring + dst) = ldg16(z_new + r * nsr + e);
}

// one workgroup per row; rows whose token does not end a region exit
__global__ __launch_bounds__(256) void append_summarize_kernel(
    const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos,
    const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ z_ring, int64_t B,
    int64_t slots, int64_t rsb, const float* __restrict__ lnw, const float* __restrict__ lnb,
    float eps, const uint16_t* __restrict__ rope, int64_t rope_rows, uint8_t* __restrict__ S,
    int64_t ssb, int64_t R_cap) {
  const int64_t r = blockIdx.x;
  const int32_t s = row_seq[r];
  const int64_t p = row_pos[r];
  if (!append_row_ok(s, p, B, rope_rows, R_cap) || (p & 7) != 7) return;  // block-uniform
  const int t = threadIdx.x >> 5, sub = threadIdx.x & 31;
  const int g = sub >> 3, c = sub & 7;
  const int64_t a = p - 7;  // the region's first token
  const int64_t off = (int64_t)s * rsb + ((a % slots) + t) * 256 + g * 64 + c * 8;
  summarize_region_block(k_ring + off, z_ring + off, rope + (a + t) * 32, lnw, lnb, eps,
                         S + (int64_t)s * ssb + (p >> 3) * 256 + g * 64 + c * 8);
}

// spans of up to this many regions run token-parallel
#ifndef S5_SUMMARY_SMALL_MAX
#define S5_SUMMARY_SMALL_MAX 1024
#endif

hipError_t launch_summarize(const SummarizeArgs& a, hipStream_t stream) {
  const int64_t nreg = a.T / 8;
  const int64_t total = a.B * nreg;
  if (total <= 0) return hipSuccess;
  if (total <= S5_SUMMARY_SMALL_MAX) {
    hipLaunchKernelGGL(summarize_small_kernel, dim3((unsigned)total), dim3(256), 0, stream,
                       (const uint16_t*)a.k, (const uint16_t*)a.z, nreg, a.t0, a.sb, a.st,
                       a.ln_w, a.ln_b, a.eps, (const uint16_t*)a.rope, (uint8_t*)a.summary,
                       a.ssb);
    return hipGetLastError();
  }
  int64_t blocks = (total + 7) / 8;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(summarize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t*)a.k, (const uint16_t*)a.z, nreg, total, a.t0, a.sb, a.st,
                     a.ln_w, a.ln_b, a.eps, (const uint16_t*)a.rope, (uint8_t*)a.summary, a.ssb);
  return hipGetLastError();
}

// One launch when no two rows share a sequence (a decode step): one
// workgroup per row (append_row_block).
__global__ __launch_bounds__(256) void append_one_per_seq_kernel(AppendArgs a) {
  __shared__ uint4 z_lds[8][32];
  __shared__ float4 ep_lds[8][32][4];
  append_row_block(a, blockIdx.x, z_lds, ep_lds);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.one_per_seq) {
    hipLaunchKernelGGL(append_one_per_seq_kernel, dim3((unsigned)a.rows), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(append_scatter_kernel, dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0,
                     stream, (const uint16_t*)a.k_new, (const uint16_t*)a.z_new, a.new_stride_row,
                     a.row_seq, a.row_pos, a.rows, (uint16_t*)a.k_ring, (uint16_t*)a.z_ring, a.B,
                     a.slots, a.ring_stride_b, a.rope_rows, a.R_cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_summarize_kernel, dim3((unsigned)a.rows), dim3(256), 0, stream,
                     a.row_seq, a.row_pos, (const uint16_t*)a.k_ring, (const uint16_t*)a.z_ring,
                     a.B, a.slots, a.ring_stride_b, a.ln_w, a.ln_b, a.eps,
                     (const uint16_t*)a.rope, a.rope_rows, (uint8_t*)a.summary, a.ssb, a.R_cap);
  return hipGetLastError();
}

}  // namespace s5
