// Device helpers shared by the gfx950 kernels of the Step-5 sparse-indexer
// path: number formats, the path's fixed exp, lane reductions over 8- and
// 16-lane groups, and MFMA operand types.
//
// Every float operation in the bit-exact steps (indexer q/k prep, region
// summary, score epilogue) must be the single IEEE operation written, so the
// library is built with -ffp-contract=off and the helpers below use explicit
// fmaf only where the arithmetic says fused multiply-add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s5 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
__host__ __device__ inline float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__host__ __device__ inline float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// fp32 -> bf16 bit pattern, nearest with ties to even (finite values).
__host__ __device__ inline uint32_t bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// the fp32 value of that bf16
__host__ __device__ inline float bf16_round(float f) {
  return __builtin_bit_cast(float, bf16_bits(f) << 16);
}

// ---------------------------------------------------------------------------
// e4m3 (OCP E4M3, bias 7, 3 mantissa bits, subnormals, largest finite 448)
// from a bf16 bit pattern (8 exponent bits, bias 127, 7 mantissa bits),
// nearest with ties to even; magnitudes from 448 up saturate to 448.
// ---------------------------------------------------------------------------
__host__ __device__ inline uint32_t e4m3_from_bf16(uint32_t h) {
  const uint32_t sign = (h >> 8) & 0x80u;
  const uint32_t a = h & 0x7fffu;
  if (a >= 0x43e0u) return sign | 0x7eu;  // |x| >= 448
  const uint32_t E = a >> 7;              // biased bf16 exponent
  const uint32_t m7 = a & 0x7fu;
  if (E >= 121u) {
    // normal in e4m3: exponent field E - 120, keep the top 3 mantissa bits and
    // round on the 4 dropped ones; a carry out of the mantissa bumps the
    // exponent, which is the right next value
    uint32_t v = ((E - 120u) << 3) | (m7 >> 4);
    const uint32_t rem = m7 & 0xfu;
    v += (rem > 8u) | ((rem == 8u) & (v & 1u));
    return sign | v;
  }
  // subnormal in e4m3 (steps of 2^-9): code = round((1.m7) * 2^(E-127) * 2^9)
  //                                         = round((128 + m7) / 2^(125 - E))
  if (E + 9u <= 125u) return sign;  // below 2^-10 (or a bf16 subnormal): rounds to 0
  const uint32_t mant = 128u | m7;
  const uint32_t sh = 125u - E;     // 5 .. 8
  uint32_t v = mant >> sh;
  const uint32_t rem = mant & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1u);
  v += (rem > half) | ((rem == half) & (v & 1u));
  return sign | v;                  // v == 8 is the smallest normal, as it should be
}

// The same two roundings by gfx950's conversion instructions, two values at a
// time (a to the low half or byte, b to the next). bf16: nearest-even, as
// bf16_bits for every finite input (fp32 denormals are kept, the default
// mode). e4m3 of a bf16 value given as fp32: the clamp to +-448 first makes
// the hardware's nearest-even conversion saturate like e4m3_from_bf16. Both
// are checked against the software forms on the GPU, over every input.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t bf16x2_hw(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
template <bool HIGH_WORD>
__device__ inline uint32_t e4m3x2_hw(float a, float b, uint32_t old) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HIGH_WORD);
}

// ---------------------------------------------------------------------------
// The path's exp: Cody & Waite's (1980) argument reduction x = n*ln2 + r,
// |r| <= ln2/2, with ln2 split in a 15-bit head and an fp32 tail; e^r from
// its degree-7 Taylor polynomial (coefficients 1/k!) in Horner form with
// fused multiply-adds; then scaling by 2^n. The argument is first clamped to
// [-87, 88] so every result is a normal float. All steps are correctly
// rounded IEEE operations, so any conforming implementation of the same
// steps gives the same bits.
// ---------------------------------------------------------------------------
__host__ __device__ inline float exp_fixed(float x) {
  x = fminf(fmaxf(x, -87.0f), 88.0f);
  const float t = x * 0x1.715476p+0f;            // fp32(1/ln 2)
  const float n = rintf(t);
  float r = fmaf(-n, 0x1.62e4p-1f, x);           // ln 2 cut to 15 significant bits
  r = fmaf(-n, 0x1.7f7d1cp-20f, r);              // fp32(ln 2 - head)
  float p = 0x1.a01a02p-13f;                     // 1/5040
  p = fmaf(p, r, 0x1.6c16c2p-10f);               // 1/720
  p = fmaf(p, r, 0x1.111112p-7f);                // 1/120
  p = fmaf(p, r, 0x1.555556p-5f);                // 1/24
  p = fmaf(p, r, 0x1.555556p-3f);                // 1/6
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

// Pairwise sum of 8 values as a halving tree (strides 4, 2, 1).
__host__ __device__ inline float pair8(const float* a) {
  const float b0 = a[0] + a[4], b1 = a[1] + a[5], b2 = a[2] + a[6], b3 = a[3] + a[7];
  const float c0 = b0 + b2, c1 = b1 + b3;
  return c0 + c1;
}

// ---------------------------------------------------------------------------
// Cross-lane moves (DPP). Control codes: quad permutations, and shifts or
// rotations within rows of 16 lanes (row_shl:n reads lane i+n, row_shr:n
// reads lane i-n, row_ror:n reads lane (i-n) mod 16).
// ---------------------------------------------------------------------------
enum : int {
  DPP_QUAD_XOR1 = 0xB1,  // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,  // quad_perm [2,3,0,1]
  DPP_ROW_SHL4 = 0x104,
  DPP_ROW_SHR4 = 0x114,
  DPP_ROW_ROR4 = 0x124,
  DPP_ROW_ROR8 = 0x128,
  DPP_ROW_ROR12 = 0x12C,
};

template <int CTRL>
__device__ inline uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Lanes 8k+c (c = 0..7) each hold s_c; every lane of the 8-lane group gets
// ((s0+s4) + (s2+s6)) + ((s1+s5) + (s3+s7)): the halving tree over the 8
// lane values. Needs all 8 lanes of the group active.
__device__ inline float sum8_lanes(float s, int lane) {
  float t = s + dpp<DPP_ROW_SHL4>(s);   // lanes c < 4: s_c + s_{c+4}
  t = t + dpp<DPP_QUAD_XOR2>(t);        // lanes c < 4: b_c + b_{c^2}
  t = t + dpp<DPP_QUAD_XOR1>(t);        // lanes c < 4: (b0+b2) + (b1+b3), addition commutes
  const float u = dpp<DPP_ROW_SHR4>(t); // lanes c >= 4 take lane c-4's total
  return (lane & 4) ? u : t;
}

// max and sum over the 16 lanes of a row; every lane of the row gets the result
__device__ inline float max16_lanes(float v) {
  v = fmaxf(v, dpp<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp<DPP_ROW_ROR4>(v));
  v = fmaxf(v, dpp<DPP_ROW_ROR8>(v));
  return v;
}
__device__ inline float sum16_lanes(float v) {
  v = v + dpp<DPP_QUAD_XOR1>(v);
  v = v + dpp<DPP_QUAD_XOR2>(v);
  v = v + dpp<DPP_ROW_ROR4>(v);
  v = v + dpp<DPP_ROW_ROR8>(v);
  return v;
}

__device__ inline float wave_uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// 8 bf16 (16 bytes) -> 8 floats
__device__ inline void unpack_bf16x8(const uint4 w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z); f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

__device__ inline uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// word 3 of a raw buffer resource on gfx9 parts (32-bit data format; no
// swizzle, no stride): reads at offsets from the record count on return zero
constexpr int RAW_RSRC3 = 0x00020000;
// a byte offset past every record count the kernels give a resource
// (at most a few hundred MB): a store there is dropped
constexpr uint32_t RAW_PAST_END = 0x7ffffff0u;

// the exact value of an e4m3 code (every e4m3 value is an fp32 value)
__device__ inline double e4m3_f64(uint8_t b) {
  return (double)__builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// A 4 x 4 transpose over (16-lane row of the wave, register) with gfx950's
// lane swaps: on return t[i] in lane 16r + c holds what t[r] held in lane
// 16i + c. (The 32-lane swap exchanges the upper half of its first operand
// with the lower half of its second; the 16-lane swap exchanges the odd
// rows of its first operand with the even rows of its second.)
__device__ inline void transpose_rows4(uint32_t (&t)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(t[0], t[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(t[1], t[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  t[0] = c[0];
  t[1] = c[1];
  t[2] = d[0];
  t[3] = d[1];
}

// 32-bit key ordered like the float score (-0 first turned into +0 by adding
// +0); every key but that of one negative NaN pattern is nonzero, and the
// selection uses 0 for "no candidate"
__device__ inline uint32_t ord_key(float s) {
  const uint32_t u = __builtin_bit_cast(uint32_t, s + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Arrival of a block at a per-unit counter after it has written its part of a
// result to global memory; true in the one block that arrives last, which may
// then read every other block's part. Each wave first waits until its own
// stores have been acknowledged by L2 (the workgroup barrier alone does not
// wait for global stores), the block synchronises, and one thread makes the
// block's stores visible device-wide (release), takes a ticket and, if last,
// drops stale cached copies (acquire). `flag` is a __shared__ int.
__device__ inline bool block_arrive_last(unsigned* counter, unsigned nblocks, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const bool last = atomicAdd(counter, 1u) == nblocks - 1u;
    if (last) __threadfence();
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

}  // namespace s5
