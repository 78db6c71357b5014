// Sparse attention for KV heads that serve 8 or 16 query heads, or a head dim
// of 192: the geometry of Step-5's own layers on the TensorFold page
// (pull request #903, "Step-5-Preview on one 256 GB Mac", the commit note
// that adds s5_attend_nax: a (row, KV group) unit, the group's 16 query heads
// as the left operand over 32 keys at a time, 192-dim heads, bf16 products
// summed in fp32, probabilities applied to the values as bf16 parts). vLLM's
// geometry rules allow 4, 8 or 16 query heads per KV head.
//
// The unit's entries (own region first, then the selected regions) and the
// fixed-order split merge are those of attn.hip. A workgroup takes one split
// and walks it in 32-token chunks (4 entries), all four waves on the same
// chunk:
//  - the chunk's K and V rows go straight from memory into LDS
//    (global_load_lds, 16 B per lane, no registers), into a ring of three
//    buffers at head dim 128 (two chunks load while one is computed) or two
//    at 192 (one). A token row's 16-byte pieces are stored in XOR-swizzled
//    slots, so that the reads below fall in distinct LDS banks. Each chunk's
//    loads are waited for by count, and the buffers are read by LDS reads
//    that wait only for themselves, so that no wait covers a later chunk;
//  - S = Q K^T on the 16x16x32 bf16 MFMA: A = the unit's query heads (MFMA
//    rows; rows past QPK are zero), B = 16 key tokens, each lane's D/4 dims
//    read from LDS as 16-byte slices; every wave computes all of S;
//  - online softmax in the log2 domain per head: output lane (n, qd) holds
//    heads 4qd..4qd+3 for token n, a head's max and sum are reductions over
//    one 16-lane row; the state is the same in every wave;
//  - O += P V on the same MFMA, each wave for a quarter of the dims: A = P
//    (heads x 32 tokens), split into a bf16 high part and the bf16 of the
//    remainder (two MFMAs, error ~2^-17 of P), through LDS to reach the
//    operand layout; B = V with tokens along the contraction, read from LDS
//    2 bytes at a time (8 tokens of one dim per lane).
// The waves' states need no merge: each holds its own dims.
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

namespace {

constexpr int MH_ENTRIES = 513;  // own region + 512 selections
// chunk buffers: with 3, two chunks load while one is computed (head dim 128,
// 62 KB of LDS: two workgroups per CU); with 2, one (head dim 192, whose
// three buffers would leave one workgroup per CU)
template <int D>
constexpr int mh_nb() { return D <= 128 ? 3 : 2; }

template <int QPK, int D>
struct MhCfg {
  static constexpr int KS = D / 32;               // QK^T MFMA steps of 32 dims
  static constexpr int NT = D / 16;               // PV output tiles of 16 dims
  static constexpr int TPW = NT / 4;              // PV tiles per wave
  static constexpr int PIECES = D / 8;            // 16-byte pieces of a token row
  static constexpr int CP = 32 * PIECES;          // pieces of a chunk's K (or V)
  static constexpr int PPT = CP / 256;            // pieces per thread per chunk
  static constexpr int PART = 2 + D;              // split state per head: m, l, o[D]
  static_assert(QPK == 4 || QPK == 8 || QPK == 16, "query heads per KV head");
  static_assert(D % 64 == 0 && PIECES % 8 == 0 && CP % 256 == 0, "head dim");
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

// 16 bytes from global memory straight into LDS: the lane's bytes land at
// lds + 16 * lane (lds the same in every lane)
__device__ inline void mh_load_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// wait until at most N of this wave's vector memory operations (loads into
// LDS included) are outstanding; they complete in issue order
template <int N>
__device__ inline void mh_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS reads of the chunk buffers. They are written by global_load_lds, and a
// compiler-generated read of them would be preceded by a wait for every
// outstanding load into LDS, the next chunks' included; these reads wait
// only for themselves (in the same statement), the chunk's own loads having
// been waited for explicitly.
__device__ inline uint32_t mh_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int N>
__device__ inline void mh_lds_read16(uint4 (&v)[N], const uint32_t (&a)[N]) {
  static_assert(N == 4 || N == 6, "reads per statement");
  if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %6\n\tds_read_b128 %1, %7\n\tds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\tds_read_b128 %4, %10\n\tds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
        : "memory");
  }
}
// eight 16-bit LDS values, zero-extended
__device__ inline void mh_lds_read2x8(uint32_t (&v)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_u16 %0, %8\n\tds_read_u16 %1, %9\n\tds_read_u16 %2, %10\n\t"
      "ds_read_u16 %3, %11\n\tds_read_u16 %4, %12\n\tds_read_u16 %5, %13\n\t"
      "ds_read_u16 %6, %14\n\tds_read_u16 %7, %15\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// slot of piece P of chunk token tt: K rows are read 16 B per lane by 8
// consecutive tokens, V rows 2 B per lane by 16 dims x 4 token groups
__device__ inline int mh_kslot(int tt, int P) { return P ^ (tt & 7); }
__device__ inline int mh_vslot(int tt, int P) { return P ^ ((tt & 7) ^ (2 * (tt >> 3))); }

}  // namespace

template <int QPK, int D>
__global__ __launch_bounds__(256) void attn_mh_kernel(
    const uint16_t* __restrict__ q, int64_t qs, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t B, int64_t kv_sb, int64_t kv_st, int64_t T_cap,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, float scale_log2, int per_split, int nsplit,
    float* __restrict__ partial, uint16_t* __restrict__ out, float* __restrict__ lse) {
  using C = MhCfg<QPK, D>;
  constexpr int NB = mh_nb<D>();
  __shared__ __align__(16) uint4 kv_lds[NB][2][C::CP];        // [buffer][K | V][slot]
  __shared__ __align__(16) uint16_t p_lds[4][2][16 * 32];     // per wave: P high, low [head][token]
  __shared__ uint32_t ids_lds[512];
  __shared__ int32_t ent_j[MH_ENTRIES + 3];                   // the split's entries: region id
  __shared__ uint8_t ent_n[MH_ENTRIES + 3];                   // and token count (0: empty)

  const int64_t unit = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, qd = lane >> 4;

  const int32_t seq = row_seq[row];
  const int64_t p = row_pos[row];
  const bool valid = seq >= 0 && seq < B && p >= 0 && p < T_cap;
  const int64_t ncand = valid ? (p >> 3) : 0;
  const int nent = valid ? 1 + (int)(ncand < 512 ? ncand : 512) : 0;
  const int e0 = split * per_split;
  const int e1 = min(e0 + per_split, nent);
  const int nch = e1 > e0 ? (e1 - e0 + 3) >> 2 : 0;
  const int32_t* sl = sel + unit * 512;
  if (nsplit == 1) {
    // unsplit (many rows): visit the selected regions in id order, as attn.hip does
    for (int i = tid; i < 512; i += 256) ids_lds[i] = (uint32_t)sl[i];
    __syncthreads();
#pragma unroll 1
    for (int kk = 2; kk <= 512; kk <<= 1)
#pragma unroll 1
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = tid + 256 * h;
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
  // the split's entries, padded to whole chunks with empty ones
  for (int e = tid; e < 4 * nch; e += 256) {
    const int ge = e0 + e;
    int32_t j = 0;
    int cnt = 0;
    if (ge < e1) {
      if (ge == 0) {
        j = (int32_t)(p >> 3);
        cnt = (int)(p & 7) + 1;
      } else {
        const int32_t s = sl[ge - 1];
        if (s >= 0 && s < ncand) {
          j = s;
          cnt = 8;
        }
      }
    }
    ent_j[e] = j;
    ent_n[e] = (uint8_t)cnt;
  }
  __syncthreads();

  const int64_t sb = valid ? (int64_t)seq * kv_sb : 0;
  const uint16_t* kb = kc + sb + (int64_t)g * D;
  const uint16_t* vb = vc + sb + (int64_t)g * D;
  const int64_t pc = valid ? p : 0;  // a token that is always in range
  // A operand of S: head n of the unit (zero past QPK), dims qd*D/4 ...
  // (loaded before the chunks, so that the waits below, which count the
  // chunks' loads, never wait for them)
  uint4 qa[C::KS];
#pragma unroll
  for (int u = 0; u < C::KS; ++u) qa[u] = make_uint4(0, 0, 0, 0);
  if (valid && n < QPK) {
    const uint16_t* qp = q + row * qs + (int64_t)(QPK * g + n) * D + qd * (D / 4);
#pragma unroll
    for (int u = 0; u < C::KS; ++u) qa[u] = ldg16(qp + 8 * u);
  }
  // chunk c into buffer bf: thread tid fills slots r * 256 + tid of K and V
  auto stage = [&](int c, int bf) {
#pragma unroll
    for (int r = 0; r < C::PPT; ++r) {
      const int s = r * 256 + tid;
      const int tt = s / C::PIECES, sg = s - tt * C::PIECES;
      const int e = 4 * c + (tt >> 3), ti = tt & 7;
      const int64_t tok = ti < (int)ent_n[e] ? 8 * (int64_t)ent_j[e] + ti : pc;
      const uint16_t* krow = kb + tok * kv_st;
      const uint16_t* vrow = vb + tok * kv_st;
      // slot sg holds piece mh_kslot(tt, sg) (an involution)
      mh_load_lds16(krow + 8 * mh_kslot(tt, sg), &kv_lds[bf][0][r * 256 + wave * 64]);
      mh_load_lds16(vrow + 8 * mh_vslot(tt, sg), &kv_lds[bf][1][r * 256 + wave * 64]);
    }
  };


  float m[4], l[4];
  f32x4 o[C::TPW];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < C::TPW; ++c) o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  uint16_t* pw_hi = p_lds[wave][0];
  uint16_t* pw_lo = p_lds[wave][1];

  // each thread issues 2 PPT loads per chunk; chunks c + 1 .. c + NB - 1 are
  // in flight while chunk c is computed
  static_assert(NB == 2 || NB == 3, "the waits below count at most one chunk in flight");
  constexpr int LPC = 2 * C::PPT;
#pragma unroll
  for (int c = 0; c < NB - 1; ++c)
    if (c < nch) stage(c, c);
#pragma unroll 1
  for (int c = 0; c < nch; ++c) {
    const int bf = c % NB;
    // this thread's loads of chunk c are done (with 3 buffers chunk c + 1's
    // may still be outstanding); after the barrier every thread's are, and
    // every wave has finished chunk c - 1, whose buffer chunk c + NB - 1 reuses
    if (NB == 3 && c + 1 < nch) mh_wait_vm<LPC>();
    else mh_wait_vm<0>();
    __syncthreads();
    if (c + NB - 1 < nch) stage(c + NB - 1, (c + NB - 1) % NB);
    const uint32_t kl = mh_lds_addr(kv_lds[bf][0]);
    const uint32_t vl = mh_lds_addr(kv_lds[bf][1]);
    // S for tokens 16 st + n of the chunk
    f32x4 acc[2];
    bool kok[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int tt = 16 * st + n;
      kok[st] = (tt & 7) < (int)ent_n[4 * c + (tt >> 3)];
      acc[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
      uint32_t ka[C::KS];
      uint4 kv[C::KS];
#pragma unroll
      for (int u = 0; u < C::KS; ++u)
        ka[u] = kl + 16u * (uint32_t)(tt * C::PIECES + mh_kslot(tt, qd * C::KS + u));
      mh_lds_read16<C::KS>(kv, ka);
#pragma unroll
      for (int u = 0; u < C::KS; ++u) acc[st] = mh_mfma(qa[u], kv[u], acc[st]);
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
    mh_wave_sync();
    const uint4 pa_hi = *reinterpret_cast<const uint4*>(pw_hi + n * 32 + 8 * qd);
    const uint4 pa_lo = *reinterpret_cast<const uint4*>(pw_lo + n * 32 + 8 * qd);
#pragma unroll
    for (int ct = 0; ct < C::TPW; ++ct) {
      const int tile = wave * C::TPW + ct;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[ct][r] *= alpha[r];
      // B: V[tokens 8qd .. 8qd+7][dim 16 tile + n]
      const int P = 2 * tile + (n >> 3), e8 = n & 7;
      uint32_t va[8], vv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int tt = 8 * qd + t;
        va[t] = vl + 2u * (uint32_t)((tt * C::PIECES + mh_vslot(tt, P)) * 8 + e8);
      }
      mh_lds_read2x8(vv, va);
      uint32_t bw[4];
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) bw[t2] = vv[2 * t2] | (vv[2 * t2 + 1] << 16);
      const uint4 bv = make_uint4(bw[0], bw[1], bw[2], bw[3]);
      o[ct] = mh_mfma(pa_hi, bv, o[ct]);
      o[ct] = mh_mfma(pa_lo, bv, o[ct]);
    }
    mh_wave_sync();
  }

  // ---- the wave's dims of every head: split state or final output
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * qd + r;
    if (h >= QPK) continue;
    const float L = l[r], M = m[r];
    if (nsplit > 1) {
      float* dst = partial + ((unit * nsplit + split) * QPK + h) * C::PART;
      if (wave == 0 && n == 0) {
        dst[0] = M;
        dst[1] = L;
      }
#pragma unroll
      for (int ct = 0; ct < C::TPW; ++ct) dst[2 + 16 * (wave * C::TPW + ct) + n] = o[ct][r];
    } else {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      uint16_t* dst = out + (row * 4 * QPK + QPK * g + h) * D;
#pragma unroll
      for (int ct = 0; ct < C::TPW; ++ct)
        dst[16 * (wave * C::TPW + ct) + n] = (uint16_t)bf16_bits(o[ct][r] * inv);
      if (lse && wave == 0 && n == 0)
        lse[row * 4 * QPK + QPK * g + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

// Merge of a unit's split states: one workgroup per (unit, head), thread d
// for dim d. Every thread reads the splits' m and l itself (the same address
// across a wave: one load each) besides its o values, all in flight at once,
// and forms M = max m_s, the weights 2^(m_s - M), L and its dim in split
// order: one memory round trip, the same result in every thread.
template <int QPK, int D>
__global__ __launch_bounds__(256) void attn_mh_merge_kernel(const float* __restrict__ partial,
                                                            int nsplit,
                                                            uint16_t* __restrict__ out,
                                                            float* __restrict__ lse) {
  using C = MhCfg<QPK, D>;
  const int64_t unit = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  const int t = threadIdx.x;
  if (t >= D) return;
  const int64_t sstride = (int64_t)QPK * C::PART;  // between a head's states of consecutive splits
  const float* st = partial + (unit * nsplit * QPK + h) * C::PART;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, st[s * sstride]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f, O = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float* sp = st + s * sstride;
    const float f = __builtin_amdgcn_exp2f(sp[0] - Mu);
    L = L + f * sp[1];
    O = O + f * sp[2 + t];
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  out[(row * 4 * QPK + QPK * g + h) * D + t] = (uint16_t)bf16_bits(O * inv);
  if (lse && t == 0)
    lse[row * 4 * QPK + QPK * g + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

// Splits: a multiple of 4 entries (one chunk) each, about S5_ATTN_MH_BLOCKS
// workgroups in all for decode; many rows run unsplit.
#ifndef S5_ATTN_MH_BLOCKS
#define S5_ATTN_MH_BLOCKS 512
#endif
static AttnPlan attn_mh_plan(int32_t rows) {
  const int64_t units = (int64_t)rows * 4;
  int64_t ns = units > 0 ? (S5_ATTN_MH_BLOCKS + units - 1) / units : 1;
  int64_t per = (MH_ENTRIES + ns - 1) / ns;
  per = (per + 3) / 4 * 4;
  if (per < 16) per = 16;
  AttnPlan a;
  a.per_split = (int32_t)per;
  a.nsplit = (int32_t)((MH_ENTRIES + per - 1) / per);
  return a;
}

size_t attn_mh_workspace_bytes(int32_t rows, int32_t qpk, int32_t head_dim) {
  const AttnPlan a = attn_mh_plan(rows);
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
  return launch_attn_merge(a.partial, pl.nsplit, a.rows, QPK, D, a.out, a.lse, stream);
}

hipError_t launch_attn_merge(const float* partial, int32_t nsplit, int32_t rows, int32_t qpk,
                             int32_t head_dim, void* out, float* lse, hipStream_t stream) {
  const dim3 grid((unsigned)rows * 4u, (unsigned)qpk);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, partial, (int)nsplit, (uint16_t*)out,
                       lse);
    return hipGetLastError();
  };
  if (head_dim == 128) {
    if (qpk == 4) return go(attn_mh_merge_kernel<4, 128>);
    if (qpk == 8) return go(attn_mh_merge_kernel<8, 128>);
    if (qpk == 16) return go(attn_mh_merge_kernel<16, 128>);
  } else if (head_dim == 192) {
    if (qpk == 4) return go(attn_mh_merge_kernel<4, 192>);
    if (qpk == 8) return go(attn_mh_merge_kernel<8, 192>);
    if (qpk == 16) return go(attn_mh_merge_kernel<16, 192>);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_mh(const AttnArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const AttnPlan pl = attn_mh_plan(a.rows);
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
