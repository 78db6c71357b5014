// Sparse attention for KV heads that serve 8 or 16 query heads, or a head dim
// of 192: the geometry of Step-5's own layers on the TensorFold page
// (pull request #903, "Step-5-Preview on one 256 GB Mac", the commit note
// that adds s5_attend_nax: a (row, KV group) unit, the group's 16 query heads
// as the left operand over 32 keys at a time, 192-dim heads, bf16 products
// summed in fp32, probabilities applied to the values as bf16 parts). vLLM's
// geometry rules allow 4, 8 or 16 query heads per KV head.
//
// The unit's entries (own region first, then the selected regions), the
// splits and the fixed-order merges are those of attn.hip. Per 32-token
// chunk, per wave:
//  - S = Q K^T on the 16x16x32 bf16 MFMA: A = the unit's query heads (MFMA
//    rows; rows past QPK are zero), B = 16 gathered key tokens; each lane
//    loads D/4 contiguous dims of one token (the MFMAs take its 16-byte
//    slices in turn, the same slices of the query), so K needs no reordering;
//  - online softmax in the log2 domain per head: output lane (n, qd) holds
//    heads 4qd..4qd+3 for token n, so a head's max and sum are reductions
//    over one 16-lane row;
//  - O += P V on the same MFMA: A = P (heads x 32 tokens), split into a bf16
//    high part and the bf16 of the remainder (two MFMAs, error ~2^-17 of P),
//    staged through LDS to reach the operand layout; B = V with tokens along
//    the contraction, which puts 8 tokens of one dim in a lane: V is staged
//    in LDS in its row layout (rows padded by one dword so the lanes of a
//    read fall in distinct banks) and read back 2 bytes at a time.
// Output lane (n, qd) of the PV MFMA holds heads 4qd..4qd+3 of dim 16c + n,
// the same heads as the softmax state it is rescaled by.
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

namespace {

constexpr int MH_ENTRIES = 513;  // own region + 512 selections

template <int QPK, int D>
struct MhCfg {
  static constexpr int KS = D / 32;               // QK^T MFMA steps of 32 dims
  static constexpr int NT = D / 16;               // PV output tiles of 16 dims
  static constexpr int PIECES = D / 8;            // 16-byte pieces of a token row
  static constexpr int VPL = 32 * PIECES / 64;    // V pieces per lane per chunk (D / 16)
  static constexpr int VROW = D + 2;              // staged V row, elements (one dword of padding)
  static constexpr int PART = 2 + D;              // split state per head: m, l, o[D]
  static_assert(QPK == 4 || QPK == 8 || QPK == 16, "query heads per KV head");
  static_assert(D % 32 == 0 && (32 * PIECES) % 64 == 0, "head dim");
};

__device__ inline void mh_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline f32x4 mh_mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <typename T>
__device__ inline T mh_pick4(int i, T a, T b, T c, T d) {
  return i < 2 ? (i == 0 ? a : b) : (i == 2 ? c : d);
}

}  // namespace

template <int QPK, int D>
__global__ __launch_bounds__(256) void attn_mh_kernel(
    const uint16_t* __restrict__ q, int64_t qs, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t B, int64_t kv_sb, int64_t kv_st, int64_t T_cap,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, float scale_log2, int per_split, int nsplit,
    float* __restrict__ partial, uint16_t* __restrict__ out, float* __restrict__ lse) {
  using C = MhCfg<QPK, D>;
  // per wave: the chunk's V rows; after the loop the waves' states (o, then m
  // and l) for the merge, which need exactly as many bytes
  __shared__ __align__(16) uint16_t v_lds[4][32 * C::VROW];
  __shared__ __align__(16) uint16_t p_lds[4][2][16 * 32];  // per wave: P high, low [head][token]
  __shared__ uint32_t ids_lds[512];

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
  const int wb = e0 + 4 * wave;
  const int niter = wb < e1 ? (e1 - wb + 15) >> 4 : 0;
  const int32_t* sl = sel + unit * 512;
  if (nsplit == 1) {
    // unsplit (many rows): visit the selected regions in id order, as attn.hip does
    for (int i = threadIdx.x; i < 512; i += 256) ids_lds[i] = (uint32_t)sl[i];
    __syncthreads();
#pragma unroll 1
    for (int kk = 2; kk <= 512; kk <<= 1)
#pragma unroll 1
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = threadIdx.x + 256 * h;
          const int pi = i ^ jj;
          if (pi > i) {
            const uint32_t a = ids_lds[i], b = ids_lds[pi];
            const bool up = (i & kk) == 0;
            if ((a > b) == up) {
              ids_lds[i] = b;
              ids_lds[pi] = a;
            }
          }
        }
        __syncthreads();
      }
    sl = reinterpret_cast<const int32_t*>(ids_lds);
  }
  // lane 4 (i % 16) + e4 describes entry wb + 16 i + e4 of this wave
  int64_t lj = 0;
  int lcnt = 0;
  auto load_table = [&](int ibase) {
    const int e = wb + 16 * (ibase + (lane >> 2)) + (lane & 3);
    lj = 0;
    lcnt = 0;
    if (e < e1) {
      if (e == 0) {
        lj = p >> 3;
        lcnt = (int)(p & 7) + 1;
      } else {
        const int32_t j = sl[e - 1];
        if (j >= 0 && j < ncand) {
          lj = j;
          lcnt = 8;
        }
      }
    }
  };
  load_table(0);

  // A operand of S: head n of the unit (zero past QPK), dims qd*D/4 ...
  uint4 qa[C::KS];
#pragma unroll
  for (int u = 0; u < C::KS; ++u) qa[u] = make_uint4(0, 0, 0, 0);
  if (valid && n < QPK) {
    const uint16_t* qp = q + row * qs + (int64_t)(QPK * g + n) * D + qd * (D / 4);
#pragma unroll
    for (int u = 0; u < C::KS; ++u) qa[u] = ldg16(qp + 8 * u);
  }
  const int64_t sb = valid ? (int64_t)seq * kv_sb : 0;
  const uint16_t* kb = kc + sb + (int64_t)g * D;
  const uint16_t* vb = vc + sb + (int64_t)g * D;
  const int64_t pc = valid ? p : 0;  // a token that is always in range

  float m[4], l[4];
  f32x4 o[C::NT];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < C::NT; ++c) o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  uint16_t* vw = v_lds[wave];
  uint16_t* pw_hi = p_lds[wave][0];
  uint16_t* pw_lo = p_lds[wave][1];

#pragma unroll 1
  for (int i = 0; i < niter; ++i) {
    if (i > 0 && (i & 15) == 0) load_table(i);
    const int src0 = 4 * (i & 15);
    int64_t jr[4];
    int cnt[4];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)lj, src0 + e4);
      const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(lj >> 32), src0 + e4);
      jr[e4] = (int64_t)(((uint64_t)hi << 32) | lo);
      cnt[e4] = __builtin_amdgcn_readlane(lcnt, src0 + e4);
    }
    // K: lane (n, qd) of tile st holds token 16 st + n, dims qd*D/4 ...
    uint4 kr[2][C::KS];
    bool kok[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int e4 = 2 * st + (n >> 3), ti = n & 7;
      kok[st] = ti < mh_pick4(e4, cnt[0], cnt[1], cnt[2], cnt[3]);
      const int64_t tok = kok[st] ? 8 * mh_pick4(e4, jr[0], jr[1], jr[2], jr[3]) + ti : pc;
      const uint16_t* kp = kb + tok * kv_st + qd * (D / 4);
#pragma unroll
      for (int u = 0; u < C::KS; ++u) kr[st][u] = ldg16(kp + 8 * u);
    }
    // V: piece x = lane + 64 v of the chunk's 32 x D/8 pieces (absent tokens
    // load the own token; their probability is 0)
    uint4 vr[C::VPL];
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const int x = lane + 64 * v;
      const int tt = x / C::PIECES, dp = x - tt * C::PIECES;
      const int e4 = tt >> 3, ti = tt & 7;
      const int64_t tok = ti < mh_pick4(e4, cnt[0], cnt[1], cnt[2], cnt[3])
                              ? 8 * mh_pick4(e4, jr[0], jr[1], jr[2], jr[3]) + ti
                              : pc;
      vr[v] = ldg16(vb + tok * kv_st + 8 * dp);
    }
    // S, then the online softmax per head (lane row qd holds heads 4qd..4qd+3)
    f32x4 acc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      acc[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < C::KS; ++u) acc[st] = mh_mfma(qa[u], kr[st][u], acc[st]);
    }
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s0 = kok[0] ? acc[0][r] * scale_log2 : -INFINITY;
      const float s1 = kok[1] ? acc[1][r] * scale_log2 : -INFINITY;
      const float cmax = max16_lanes(fmaxf(s0, s1));
      const float mnew = fmaxf(m[r], cmax);
      const float mu = (mnew == -INFINITY) ? 0.f : mnew;
      alpha[r] = __builtin_amdgcn_exp2f(m[r] - mu);
      const float p0 = __builtin_amdgcn_exp2f(s0 - mu);
      const float p1 = __builtin_amdgcn_exp2f(s1 - mu);
      l[r] = l[r] * alpha[r] + sum16_lanes(p0 + p1);
      m[r] = mnew;
      // P as bf16 high part and bf16 of the remainder, [head][token]
      const int h = 4 * qd + r;
      const uint32_t h0 = bf16_bits(p0), h1 = bf16_bits(p1);
      pw_hi[h * 32 + n] = (uint16_t)h0;
      pw_hi[h * 32 + 16 + n] = (uint16_t)h1;
      pw_lo[h * 32 + n] = (uint16_t)bf16_bits(p0 - __builtin_bit_cast(float, h0 << 16));
      pw_lo[h * 32 + 16 + n] = (uint16_t)bf16_bits(p1 - __builtin_bit_cast(float, h1 << 16));
    }
    // V rows into LDS (4-byte stores: the padded rows are 4-byte aligned)
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const int x = lane + 64 * v;
      const int tt = x / C::PIECES, dp = x - tt * C::PIECES;
      uint32_t* dst = reinterpret_cast<uint32_t*>(vw + tt * C::VROW + 8 * dp);
      dst[0] = vr[v].x;
      dst[1] = vr[v].y;
      dst[2] = vr[v].z;
      dst[3] = vr[v].w;
    }
    mh_wave_sync();
    const uint4 pa_hi = *reinterpret_cast<const uint4*>(pw_hi + n * 32 + 8 * qd);
    const uint4 pa_lo = *reinterpret_cast<const uint4*>(pw_lo + n * 32 + 8 * qd);
#pragma unroll
    for (int c = 0; c < C::NT; ++c) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[c][r] *= alpha[r];
      // B: V[tokens 8qd .. 8qd+7][dim 16c + n]
      const uint16_t* vp = vw + (8 * qd) * C::VROW + 16 * c + n;
      uint32_t bw[4];
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2)
        bw[t2] = (uint32_t)vp[(2 * t2) * C::VROW] | ((uint32_t)vp[(2 * t2 + 1) * C::VROW] << 16);
      const uint4 bv = make_uint4(bw[0], bw[1], bw[2], bw[3]);
      o[c] = mh_mfma(pa_hi, bv, o[c]);
      o[c] = mh_mfma(pa_lo, bv, o[c]);
    }
    mh_wave_sync();
  }

  // ---- merge the four waves (fixed order), through the V staging area
  __syncthreads();
  float* mo = reinterpret_cast<float*>(&v_lds[0][0]);          // [wave][16 heads][D]
  float* ml = mo + 4 * 16 * D;                                  // [wave][m | l][16 heads]
#pragma unroll
  for (int c = 0; c < C::NT; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) mo[(wave * 16 + 4 * qd + r) * D + 16 * c + n] = o[c][r];
  if (n == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ml[(wave * 2 + 0) * 16 + 4 * qd + r] = m[r];
      ml[(wave * 2 + 1) * 16 + 4 * qd + r] = l[r];
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < QPK * D; x += 256) {
    const int h = x / D, d = x - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[(w * 2) * 16 + h]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(ml[(w * 2) * 16 + h] - Mu);
      L = L + f * ml[(w * 2 + 1) * 16 + h];
      O = O + f * mo[(w * 16 + h) * D + d];
    }
    if (nsplit > 1) {
      float* dst = partial + ((unit * nsplit + split) * QPK + h) * C::PART;
      if (d == 0) {
        dst[0] = M;
        dst[1] = L;
      }
      dst[2 + d] = O;
    } else {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      out[(row * 4 * QPK + QPK * g + h) * D + d] = (uint16_t)bf16_bits(O * inv);
      if (lse && d == 0)
        lse[row * 4 * QPK + QPK * g + h] =
            L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

// Merge of a unit's split states in split order: thread x takes output
// (head, dim) pairs; every split's m and l are read by all threads of a head.
template <int QPK, int D>
__global__ __launch_bounds__(256) void attn_mh_merge_kernel(const float* __restrict__ partial,
                                                            int nsplit,
                                                            uint16_t* __restrict__ out,
                                                            float* __restrict__ lse) {
  using C = MhCfg<QPK, D>;
  const int64_t unit = blockIdx.x;
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  const float* st = partial + unit * (int64_t)nsplit * QPK * C::PART;
  for (int x = threadIdx.x; x < QPK * D; x += 256) {
    const int h = x / D, d = x - h * D;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, st[(s * QPK + h) * C::PART]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float* sp = st + (s * QPK + h) * C::PART;
      const float f = __builtin_amdgcn_exp2f(sp[0] - Mu);
      L = L + f * sp[1];
      O = O + f * sp[2 + d];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    out[(row * 4 * QPK + QPK * g + h) * D + d] = (uint16_t)bf16_bits(O * inv);
    if (lse && d == 0)
      lse[row * 4 * QPK + QPK * g + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
  }
}

size_t attn_mh_workspace_bytes(int32_t rows, int32_t qpk, int32_t head_dim) {
  const AttnPlan a = attn_plan(rows);
  if (a.nsplit <= 1) return 0;
  return (size_t)rows * 4 * a.nsplit * qpk * (2 + head_dim) * sizeof(float);
}

template <int QPK, int D>
static hipError_t launch_mh(const AttnArgs& a, const AttnPlan& pl, hipStream_t stream) {
  const unsigned units = (unsigned)a.rows * 4u;
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  hipLaunchKernelGGL((attn_mh_kernel<QPK, D>), dim3(units, (unsigned)pl.nsplit), dim3(256), 0,
                     stream, (const uint16_t*)a.q, a.q_stride_row, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.B, a.kv_sb, a.kv_st, a.T_cap, a.sel, a.row_seq,
                     a.row_pos, scale_log2, pl.per_split, pl.nsplit, a.partial, (uint16_t*)a.out,
                     a.lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  hipLaunchKernelGGL((attn_mh_merge_kernel<QPK, D>), dim3(units), dim3(256), 0, stream,
                     (const float*)a.partial, pl.nsplit, (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

hipError_t launch_attn_mh(const AttnArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const AttnPlan pl = attn_plan(a.rows);
  if (a.head_dim == 128) {
    if (a.qpk == 4) return launch_mh<4, 128>(a, pl, stream);
    if (a.qpk == 8) return launch_mh<8, 128>(a, pl, stream);
    if (a.qpk == 16) return launch_mh<16, 128>(a, pl, stream);
  } else if (a.head_dim == 192) {
    if (a.qpk == 4) return launch_mh<4, 192>(a, pl, stream);
    if (a.qpk == 8) return launch_mh<8, 192>(a, pl, stream);
    if (a.qpk == 16) return launch_mh<16, 192>(a, pl, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace s5
