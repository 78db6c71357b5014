// Sparse attention over a row's selected regions plus its own region.
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"): the indexer commit
// note attends over the selected regions and the row's own region; the
// attention commit note splits a row's keys across workers whose online
// softmax states are merged in a fixed order. The split here is the same
// idea cut for gfx950: a (row, KV head) unit's list of 513 entries (its own
// region first, then the 512 selected regions) is cut into splits of
// `per_split` entries, one 256-thread workgroup each; inside a workgroup the
// four waves take 4-entry chunks (32 tokens) in turn; wave states merge in
// wave order, split states merge in split order. Results are therefore
// independent of scheduling.
//
// Per 32-token chunk, per wave:
//  - QK^T with the 16x16x32 bf16 MFMA: A = the unit's 4 query heads (MFMA
//    rows 0..3, the rest zero), B = 16 gathered key tokens; each lane loads
//    64 contiguous bytes (dims 32q..32q+31) of one token, the four MFMAs take
//    its 16-byte slices in turn, the same for both operands;
//  - online softmax in the log2 domain (scores scaled by scale*log2(e), hw
//    exp2), running max and sum per head kept wave-uniform;
//  - PV on the vector units: lane (n, q) accumulates dims 8n..8n+7 of the
//    four heads over tokens q, q+4, q+8, ..., reading V rows with 16-byte
//    loads (16 lanes cover a 256-byte row) and P from LDS.
// Decode units are few (rows x 4), so they get many splits to spread the
// gather over the GPU; prefill units are many and run unsplit.
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

constexpr int AT_ENTRIES = 513;  // own region + 512 selections
constexpr int AT_PART = 130;     // m, l, o[128] per head in a split state

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void attn_kernel(
    const uint16_t* __restrict__ q, int64_t qs, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t B, int64_t kv_sb, int64_t kv_st, int64_t T_cap,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, float scale_log2, int per_split, int nsplit,
    float* __restrict__ partial, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ float4 p_lds[4][32];            // per wave: P of 32 tokens, 4 heads each
  __shared__ float o_lds[4][4][4][128];      // [wave][token slot][head][dim]
  __shared__ float ml_lds[4][2][4];          // [wave][m | l][head]

  const int64_t unit = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;

  const int32_t seq = row_seq[row];
  const int64_t p = row_pos[row];
  const bool valid = seq >= 0 && seq < B && p >= 0 && p < T_cap;
  const int64_t ncand = valid ? (p >> 3) : 0;
  const int nent = valid ? 1 + (int)(ncand < 512 ? ncand : 512) : 0;
  const int e0 = split * per_split;
  const int e1 = min(e0 + per_split, nent);

  uint4 qa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qa[i] = make_uint4(0, 0, 0, 0);
  if (valid && n < 4) {
    const uint16_t* qp = q + row * qs + (4 * g + n) * 128 + 32 * qd;
#pragma unroll
    for (int i = 0; i < 4; ++i) qa[i] = ldg16(qp + 8 * i);
  }
  const int64_t sb = valid ? (int64_t)seq * kv_sb : 0;
  const uint16_t* kb = kc + sb + g * 128;
  const uint16_t* vb = vc + sb + g * 128;
  const int32_t* sl = sel + unit * 512;
  const int64_t pc = valid ? p : 0;  // a token that is always in range

  float m_run[4], l_run[4], o[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[r][i] = 0.f;
  }

  for (int ec = e0 + wave * 4; ec < e1; ec += 16) {
    int64_t jr[4];
    int cnt[4];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int e = ec + e4;
      jr[e4] = 0;
      cnt[e4] = 0;
      if (e < e1) {
        if (e == 0) {
          jr[e4] = p >> 3;
          cnt[e4] = (int)(p & 7) + 1;
        } else {
          const int32_t j = sl[e - 1];
          if (j >= 0 && j < ncand) {
            jr[e4] = j;
            cnt[e4] = 8;
          }
        }
      }
    }
    uint4 kr[2][4], vr[8];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int tt = 16 * st + n;
      const int e4 = tt >> 3, ti = tt & 7;
      const int64_t tok = (ti < cnt[e4]) ? 8 * jr[e4] + ti : pc;
      const uint16_t* kp = kb + tok * kv_st + 32 * qd;
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[st][i] = ldg16(kp + 8 * i);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e4 = k >> 1, ti = 4 * (k & 1) + qd;
      const int64_t tok = (ti < cnt[e4]) ? 8 * jr[e4] + ti : pc;
      vr[k] = ldg16(vb + tok * kv_st + 8 * n);
    }

    f32x4 acc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      acc[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[st] = mfma_bf16(qa[i], kr[st][i], acc[st]);
    }
    // lanes 0..15: acc[st][r] = score of head r with token 16*st + n
    float sv[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int tt = 16 * st + n;
      const bool ok = (tt & 7) < cnt[tt >> 3];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[st][r] = ok ? acc[st][r] * scale_log2 : -INFINITY;
    }
    float alpha[4], pv[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float cmax = wave_uniform(max16_lanes(fmaxf(sv[0][r], sv[1][r])));
      const float mnew = fmaxf(m_run[r], cmax);
      const float mu = (mnew == -INFINITY) ? 0.f : mnew;
      alpha[r] = __builtin_amdgcn_exp2f(m_run[r] - mu);
      pv[0][r] = __builtin_amdgcn_exp2f(sv[0][r] - mu);
      pv[1][r] = __builtin_amdgcn_exp2f(sv[1][r] - mu);
      const float psum = wave_uniform(sum16_lanes(pv[0][r] + pv[1][r]));
      l_run[r] = l_run[r] * alpha[r] + psum;
      m_run[r] = mnew;
    }
    if (qd == 0) {
      p_lds[wave][n] = make_float4(pv[0][0], pv[0][1], pv[0][2], pv[0][3]);
      p_lds[wave][16 + n] = make_float4(pv[1][0], pv[1][1], pv[1][2], pv[1][3]);
    }
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) o[r][i] *= alpha[r];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 pw = p_lds[wave][4 * k + qd];
      float vf[8];
      unpack_bf16x8(vr[k], vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[0][i] = fmaf(pw.x, vf[i], o[0][i]);
        o[1][i] = fmaf(pw.y, vf[i], o[1][i]);
        o[2][i] = fmaf(pw.z, vf[i], o[2][i]);
        o[3][i] = fmaf(pw.w, vf[i], o[3][i]);
      }
    }
    wave_lds_sync();
  }

  // ---- merge the four waves (fixed order)
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ml_lds[wave][0][r] = m_run[r];
      ml_lds[wave][1][r] = l_run[r];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float4* dst = reinterpret_cast<float4*>(&o_lds[wave][qd][r][8 * n]);
    dst[0] = make_float4(o[r][0], o[r][1], o[r][2], o[r][3]);
    dst[1] = make_float4(o[r][4], o[r][5], o[r][6], o[r][7]);
  }
  __syncthreads();
  const int r = threadIdx.x >> 6;
  const int d0 = 2 * (threadIdx.x & 63);
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][0][r]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float f = __builtin_amdgcn_exp2f(ml_lds[w][0][r] - Mu);
    L = L + f * ml_lds[w][1][r];
    const float s0 = ((o_lds[w][0][r][d0] + o_lds[w][1][r][d0]) + o_lds[w][2][r][d0]) + o_lds[w][3][r][d0];
    const float s1 = ((o_lds[w][0][r][d0 + 1] + o_lds[w][1][r][d0 + 1]) + o_lds[w][2][r][d0 + 1]) +
                     o_lds[w][3][r][d0 + 1];
    O0 = O0 + f * s0;
    O1 = O1 + f * s1;
  }
  if (nsplit == 1) {
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const uint32_t packed = bf16_bits(O0 * inv) | (bf16_bits(O1 * inv) << 16);
    *reinterpret_cast<uint32_t*>(out + (row * 16 + 4 * g + r) * 128 + d0) = packed;
    if (lse && d0 == 0) lse[row * 16 + 4 * g + r] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
  } else {
    float* dst = partial + ((unit * nsplit + split) * 4 + r) * AT_PART;
    if (d0 == 0) {
      dst[0] = M;
      dst[1] = L;
    }
    dst[2 + d0] = O0;
    dst[3 + d0] = O1;
  }
}

// Merge of a unit's split states, in split order. Wave r handles head r:
// lane s reads split s's (m, l) (64 splits at most), the wave reduces max and
// weighted sum, and the weights go through LDS to the o pass, where lane d
// accumulates dims 2d, 2d+1 over the splits in order with loads kept in flight.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ partial,
                                                         int nsplit, uint16_t* __restrict__ out,
                                                         float* __restrict__ lse) {
  __shared__ float f_lds[4][64];
  const int64_t unit = blockIdx.x;
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  const int r = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = 2 * lane;
  const float* base = partial + (unit * nsplit * 4 + r) * AT_PART;  // split s at + s*4*AT_PART
  const bool have = lane < nsplit;
  const float ms = have ? base[(int64_t)lane * 4 * AT_PART] : -INFINITY;
  const float ls = have ? base[(int64_t)lane * 4 * AT_PART + 1] : 0.f;
  float M = ms;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float Mu = (M == -INFINITY) ? 0.f : M;
  const float f = have ? __builtin_amdgcn_exp2f(ms - Mu) : 0.f;
  float L = f * ls;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
  f_lds[r][lane] = f;
  __syncthreads();
  float O0 = 0.f, O1 = 0.f;
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float2*>(base + (int64_t)(s + u) * 4 * AT_PART + 2 + d0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      O0 = O0 + f_lds[r][s + u] * v[u].x;
      O1 = O1 + f_lds[r][s + u] * v[u].y;
    }
  }
  for (; s < nsplit; ++s) {
    const float2 v = *reinterpret_cast<const float2*>(base + (int64_t)s * 4 * AT_PART + 2 + d0);
    O0 = O0 + f_lds[r][s] * v.x;
    O1 = O1 + f_lds[r][s] * v.y;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const uint32_t packed = bf16_bits(O0 * inv) | (bf16_bits(O1 * inv) << 16);
  *reinterpret_cast<uint32_t*>(out + (row * 16 + 4 * g + r) * 128 + d0) = packed;
  if (lse && lane == 0) lse[row * 16 + 4 * g + r] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

AttnPlan attn_plan(int32_t rows) {
  const int64_t units = (int64_t)rows * 4;
  int64_t ns = units > 0 ? (4096 + units - 1) / units : 1;
  int64_t per = (AT_ENTRIES + ns - 1) / ns;
  per = (per + 15) / 16 * 16;
  if (per < 16) per = 16;
  AttnPlan a;
  a.per_split = (int32_t)per;
  a.nsplit = (int32_t)((AT_ENTRIES + per - 1) / per);
  return a;
}

size_t attn_partial_bytes(int32_t rows) {
  const AttnPlan a = attn_plan(rows);
  if (a.nsplit <= 1) return 0;
  return (size_t)rows * 4 * a.nsplit * 4 * AT_PART * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const AttnPlan pl = attn_plan(a.rows);
  const unsigned units = (unsigned)a.rows * 4u;
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  hipLaunchKernelGGL(attn_kernel, dim3(units, (unsigned)pl.nsplit), dim3(256), 0, stream,
                     (const uint16_t*)a.q, a.q_stride_row, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.B, a.kv_sb, a.kv_st, a.T_cap, a.sel, a.row_seq,
                     a.row_pos, scale_log2, pl.per_split, pl.nsplit, a.partial, (uint16_t*)a.out,
                     a.lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(units), dim3(256), 0, stream,
                     (const float*)a.partial, pl.nsplit, (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

}  // namespace s5
