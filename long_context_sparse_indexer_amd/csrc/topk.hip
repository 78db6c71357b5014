// Top-512 region selection per (row, KV group).
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// keep the top 512 regions by (-score, id), ascending: best score first,
// equal scores by the smaller region id. Fewer than 512 candidates keep all.
//
// Input: per candidate either the score kernel's exact score (few rows) or an
// interval [lo, hi] holding the exact score (many rows). One 1024-thread
// workgroup takes a chunk of up to 16,384 candidates of one (row, group);
// thread t holds the keys of candidates t, t + 1024, ... in registers
// (scores mapped to 32-bit keys that order like the scores, -0 taken as +0;
// absent candidates get key 0, below every real key).
//   1. threshold: a thread's keys form 4 groups (keys k, k + 4, k + 8,
//      k + 12); each wave finds, by a bitwise search over ballots, a lower
//      bound of the 32nd largest of its 256 group maxima of the lower keys
//      (its top 16 bits); tau = the least of the 16 waves' values. At least
//      32 groups of every wave, 512 in all, hold a lower key >= tau, so at
//      least K = min(512, candidates) lower bounds reach tau and the K-th
//      largest lower bound is >= tau;
//   2. survivors C = the candidates whose upper key reaches tau. C holds the
//      exact top K: each of those has hi >= exact score >= K-th largest exact
//      score >= K-th largest lo >= tau. Typically |C| is 600..1,000;
//   3. (intervals) every member of C is rescored exactly on the fp64
//      matrix cores, 16 survivors per instruction chain (rescore_survivors);
//   4. the best K of C by (-exact score, id): a bitonic sort of the
//      composites (key << 32 | ~id), one per thread, 512 or 1,024 wide, or,
//      for a larger C (heavy ties), a radix select followed by a bitonic sort
//      of 512.
// A C too large to sort directly (heavy ties) is first cut: the lower keys
// >= tau include the K largest, so a radix select over just those gives T =
// the top 22 bits of the K-th largest lower key (T <= that key), and C is
// cut to the candidates whose upper key reaches T (the same argument holds).
// Candidate ranges past 16,384 are cut into chunks: each chunk keeps its
// exact best 512, sorted; the last chunk of a (row, group) to finish (an
// arrival counter per unit, zeroed by the query prep of the same call)
// merges the chunk lists pairwise.
//
// The radix select (step 4 for a large C) finds the boundary in 3 passes
// (11, 11, 10 bits): a key prefix P under a mask, such that keys above P are
// all taken and `need` keys with prefix P are taken in list order; the
// passes stop early when the boundary bin is taken whole. The bins are
// scanned by all threads at once (two bins each, a block-wide scan).
//
// Prompt chunks take topk_fused4_kernel (below): four units per workgroup,
// their intervals computed in place, thresholds, survivors and sorts done
// for the four units side by side.
#include "device.hpp"
#include "exact.hpp"
#include "interval.hpp"
#include "launch.hpp"
#include "region_block.hpp"

namespace s5 {

constexpr int TK = 512;
constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int64_t TK_MAX_N = 16384;
constexpr int TK_BINS = 2048;
constexpr int TK_PER = (int)(TK_MAX_N / TK_THREADS);  // keys per thread in registers
constexpr int TK_SORT = 1024;                           // survivors sorted directly up to this

__device__ inline float key_score(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}
__device__ inline unsigned long long compose(uint32_t key, int32_t id) {
  return ((unsigned long long)key << 32) | (uint32_t)(~(uint32_t)id);
}

struct TkShared {
  uint32_t* keys;           // [nmax]
  int32_t* ids;             // [nmax]
  uint32_t* hist;           // [TK_BINS]
  uint32_t* misc;           // [64]
  unsigned long long* out;  // [TK]
  unsigned long long* xb;   // [2 * TK_SORT] bitonic exchange
};

__host__ __device__ inline size_t tk_smem_bytes(int nmax) {
  return (size_t)TK * 8 + (size_t)2 * TK_SORT * 8 + (size_t)(TK_BINS + 64) * 4 +
         (size_t)nmax * 8;
}

__device__ inline TkShared carve(unsigned char* base, int nmax) {
  TkShared s;
  s.out = reinterpret_cast<unsigned long long*>(base);
  s.xb = s.out + TK;
  s.hist = reinterpret_cast<uint32_t*>(s.xb + 2 * TK_SORT);
  s.misc = s.hist + TK_BINS;
  s.keys = s.misc + 64;
  s.ids = reinterpret_cast<int32_t*>(s.keys + nmax);
  return s;
}

// A lower bound of the k-th largest of the wave's 4 x 64 values (1 <= k <=
// 256), the same in every lane: the largest r with at least k values >= r,
// built bit by bit from the top over the 16 high bits (the low 16 stay 0).
__device__ inline uint32_t wave_kth_largest4(const uint32_t (&v)[4], int k) {
  uint32_t r = 0;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t c = r | (1u << b);
    const int cnt = __popcll(__ballot(v[0] >= c)) + __popcll(__ballot(v[1] >= c)) +
                    __popcll(__ballot(v[2] >= c)) + __popcll(__ballot(v[3] >= c));
    if (cnt >= k) r = c;
  }
  return r;
}

__device__ inline uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
// this lane's bit of a wave-uniform lane mask, without vector instructions
__device__ inline bool lane_in(unsigned long long m) {
  return __builtin_amdgcn_inverse_ballot_w64(m);
}

// exclusive scan of v over the 1024 threads (scratch: misc[0..47]); *total gets the sum
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* misc, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) misc[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const uint32_t t = lane < TK_WAVES ? misc[lane] : 0u;
    uint32_t s = t;
#pragma unroll
    for (int o = 1; o < TK_WAVES; o <<= 1) {
      const uint32_t y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < TK_WAVES) misc[16 + lane] = s - t;
    if (lane == TK_WAVES - 1) misc[32] = s;
  }
  __syncthreads();
  const uint32_t r = misc[16 + wave] + x - v;
  *total = misc[32];
  __syncthreads();
  return r;
}

struct Boundary {
  uint32_t P, mask, need;
  uint32_t cnt;  // keys with (k & mask) == P (>= need)
};

// Radix select over keys[0..N), 1 <= K <= N: keys with (k & mask) > P are
// the K - need best; `need` more come from the keys with (k & mask) == P.
// With fewer than 3 passes P holds the K-th best key's top bits only (and
// the passes do not stop early).
__device__ Boundary radix_boundary(const TkShared& sm, int N, int K, int passes = 3) {
  const int tid = threadIdx.x;
  uint32_t P = 0, mask = 0, need = (uint32_t)K;
  const int shifts[3] = {21, 10, 0};
  const int bits[3] = {11, 11, 10};
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = shifts[pass];
    const uint32_t nb = 1u << bits[pass];
    for (int i = tid; i < (int)nb; i += TK_THREADS) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += TK_THREADS) {
      const uint32_t k = sm.keys[i];
      if ((k & mask) == P) atomicAdd(&sm.hist[(k >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    {
      // thread t owns bins nb-1-2t and nb-2-2t (two per thread, highest
      // first); an exclusive scan over threads gives the count above them,
      // and the thread whose bins hold the need-th best key reports it
      const int b_hi = (int)nb - 1 - 2 * tid, b_lo = b_hi - 1;
      const uint32_t c_hi = b_hi >= 0 ? sm.hist[b_hi] : 0u;
      const uint32_t c_lo = b_lo >= 0 ? sm.hist[b_lo] : 0u;
      uint32_t tot;
      uint32_t above = block_excl_scan(c_hi + c_lo, sm.misc, &tot);
      if (b_hi >= 0 && above < need && above + c_hi >= need) {
        sm.misc[48] = (uint32_t)b_hi;
        sm.misc[49] = need - above;
        sm.misc[50] = c_hi;
      }
      above += c_hi;
      if (b_lo >= 0 && above < need && above + c_lo >= need) {
        sm.misc[48] = (uint32_t)b_lo;
        sm.misc[49] = need - above;
        sm.misc[50] = c_lo;
      }
    }
    __syncthreads();
    const uint32_t digit = sm.misc[48], nneed = sm.misc[49], cnt = sm.misc[50];
    P |= digit << shift;
    mask |= (nb - 1) << shift;
    need = nneed;
    __syncthreads();
    if (passes == 3 && need == cnt) break;
  }
  Boundary bd;
  bd.P = P;
  bd.mask = mask;
  bd.need = need;
  bd.cnt = sm.misc[50];
  __syncthreads();
  return bd;
}

// keys/ids[0..N) -> sm.out[0..K): the best K by (key, then smaller id), in
// any order, N > K >= 1. Keys above the boundary are all taken; when more
// keys equal the K-th best key than are needed, a second radix select over
// their ids (as ~id) takes the smallest ids. sm.keys is overwritten.
__device__ void collect_best(const TkShared& sm, int N, int K) {
  const int tid = threadIdx.x;
  const Boundary bd = radix_boundary(sm, N, K);
  // the passes ran to the full key (mask all ones) unless the boundary bin
  // was taken whole, so only then can equal keys outnumber the need
  const bool tie = bd.cnt > bd.need;
  const int seg = (N + TK_THREADS - 1) / TK_THREADS;
  const int i0 = min(N, tid * seg), i1 = min(N, i0 + seg);
  uint32_t ngt = 0, neq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t m = sm.keys[i] & bd.mask;
    ngt += m > bd.P;
    neq += m == bd.P;
  }
  uint32_t tot;
  uint32_t gt_off = block_excl_scan(ngt, sm.misc, &tot);
  uint32_t eq_off = block_excl_scan(neq, sm.misc, &tot);
  const uint32_t eq_base = (uint32_t)K - bd.need;
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = sm.keys[i];
    const uint32_t m = k & bd.mask;
    if (m < bd.P) continue;
    if (m > bd.P) {
      sm.out[gt_off++] = compose(k, sm.ids[i]);
    } else if (!tie) {
      sm.out[eq_base + eq_off++] = compose(k, sm.ids[i]);
    }
  }
  if (tie) {  // block-uniform
    // keys equal to P = the K-th best key: rank them by ~id (ids are
    // distinct, so the select ends exact); every other entry drops out as 0
    __syncthreads();
    for (int i = i0; i < i1; ++i)
      sm.keys[i] = sm.keys[i] == bd.P ? ~(uint32_t)sm.ids[i] : 0u;
    __syncthreads();
    const Boundary b2 = radix_boundary(sm, N, (int)bd.need);
    uint32_t nsel = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = sm.keys[i];
      nsel += k != 0u && (k & b2.mask) >= b2.P;
    }
    uint32_t off = block_excl_scan(nsel, sm.misc, &tot);
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = sm.keys[i];
      if (k != 0u && (k & b2.mask) >= b2.P) sm.out[eq_base + off++] = compose(bd.P, (int32_t)~k);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Bitonic network, one composite per thread; the thread's index i in the
// sorted group is its thread index within the group (groups are whole
// waves). Stage (K, J): compare with element i ^ J and keep the larger where
// the K-block runs descending and i is the lower index of the pair (or
// neither), else the smaller. Which lanes keep the larger is a lane mask
// known at compile time (or per wave once K >= 64), so a stage is a 64-bit
// compare into a lane mask, a scalar xor, and two selects. Partners closer
// than 64 are in the wave: DPP for 1, 2, 8, a swizzle for 4, 16, a lane
// permute for 32; farther ones go through xb (2 x stride slots, alternated
// so one barrier per stage suffices). Every thread of the block runs the
// stages (the barriers); inactive waves exchange nothing.
// ---------------------------------------------------------------------------
struct BitonicCtx {
  int i;                   // index in the group
  int iw;                  // index of the wave's lane 0 in the group (wave-uniform)
  unsigned long long* xb;  // 2 x stride slots
  int stride;
  bool active;
  int flip;
};

__host__ __device__ constexpr unsigned long long lanes_agree(int J, int K) {
  unsigned long long m = 0;
  for (int l = 0; l < 64; ++l)
    if (((l & J) == 0) == ((l & K) == 0)) m |= 1ull << l;
  return m;
}
__host__ __device__ constexpr unsigned long long lanes_clear(int J) {
  unsigned long long m = 0;
  for (int l = 0; l < 64; ++l)
    if ((l & J) == 0) m |= 1ull << l;
  return m;
}

template <int J>
__device__ inline uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (4 << 10));    // xor 4
  } else if constexpr (J == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true); // row_ror:8
  } else if constexpr (J == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (16 << 10));   // xor 16
  } else {
    // gfx950's 32-lane swap of the value with itself: the first result holds
    // the lower half twice, the second the upper half twice (no LDS round
    // trip, unlike a bpermute)
    static_assert(J == 32, "lane_xor: J must be a power of two below 64");
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() >> 5) ? s[0] : s[1];
  }
}

template <int K, int J>
__device__ inline unsigned long long bitonic_stage(unsigned long long v, BitonicCtx& c) {
  unsigned long long p, tm;  // partner, lanes that keep the larger
  if constexpr (J >= 64) {
    unsigned long long* b = c.xb + c.stride * c.flip;
    c.flip ^= 1;
    if (c.active) b[c.i] = v;
    __syncthreads();
    p = c.active ? b[c.i ^ J] : 0ull;
    tm = (((c.iw & J) == 0) == ((c.iw & K) == 0)) ? ~0ull : 0ull;
  } else {
    p = ((unsigned long long)lane_xor<J>((uint32_t)(v >> 32)) << 32) | lane_xor<J>((uint32_t)v);
    if constexpr (K < 64) tm = lanes_agree(J, K);
    else tm = ((c.iw & K) == 0) ? lanes_clear(J) : ~lanes_clear(J);
  }
  return lane_in(~(__ballot(v > p) ^ tm)) ? v : p;
}

// stages J, J/2, ..., 1 of merge size K
template <int K, int J>
struct BitonicMerge {
  __device__ static inline unsigned long long run(unsigned long long v, BitonicCtx& c) {
    v = bitonic_stage<K, J>(v, c);
    return BitonicMerge<K, J / 2>::run(v, c);
  }
};
template <int K>
struct BitonicMerge<K, 0> {
  __device__ static inline unsigned long long run(unsigned long long v, BitonicCtx&) { return v; }
};
// full sort of blocks of K (descending where (i & K) == 0)
template <int K>
struct BitonicSort {
  __device__ static inline unsigned long long run(unsigned long long v, BitonicCtx& c) {
    v = BitonicSort<K / 2>::run(v, c);
    return BitonicMerge<K, K / 2>::run(v, c);
  }
};
template <>
struct BitonicSort<1> {
  __device__ static inline unsigned long long run(unsigned long long v, BitonicCtx&) { return v; }
};

__device__ inline BitonicCtx bitonic_ctx(int i, unsigned long long* xb, int stride, bool active) {
  BitonicCtx c;
  c.i = i;
  c.iw = __builtin_amdgcn_readfirstlane(i & ~63);
  c.xb = xb;
  c.stride = stride;
  c.active = active;
  c.flip = 0;
  return c;
}

// Composites v (one per thread of the first NS threads, 0 elsewhere) sorted
// best first: thread t < NS returns rank t.
template <int NS>
__device__ inline unsigned long long sort_desc(unsigned long long v, const TkShared& sm) {
  BitonicCtx c = bitonic_ctx((int)threadIdx.x, sm.xb, NS, (int)threadIdx.x < NS);
  return BitonicSort<NS>::run(v, c);
}

// ---------------------------------------------------------------------------

__device__ void merge_lists(const unsigned long long* __restrict__ src, int nchunks, int64_t ncand,
                            int64_t unit, unsigned char* smem, int32_t* __restrict__ sel_ids,
                            float* __restrict__ sel_scores);

__device__ inline void unit_row(const int32_t* row_seq, const int64_t* row_pos, int64_t B,
                                int64_t R_cap, int64_t pos_limit, int64_t row, int32_t* seq,
                                int64_t* ncand) {
  const int32_t s = row_seq[row];
  const int64_t p = row_pos[row];
  const bool ok = !(s < 0 || s >= B || p < 0 || p >= pos_limit || (p >> 3) > R_cap);
  *seq = ok ? s : -1;
  *ncand = ok ? (p >> 3) : 0;
}

// the rank-t composite v (rank t < K), written as id and score
__device__ inline void write_rank_at(unsigned long long v, int t, int K, int64_t unit,
                                     int32_t* sel_ids, float* sel_scores) {
  const bool have = t < K;
  sel_ids[unit * TK + t] = have ? (int32_t)(~(uint32_t)v) : -1;
  if (sel_scores) sel_scores[unit * TK + t] = have ? key_score((uint32_t)(v >> 32)) : 0.0f;
}
// thread t < 512 holds the rank-t composite v
__device__ inline void write_rank(unsigned long long v, int K, int64_t unit, int32_t* sel_ids,
                                  float* sel_scores) {
  if ((int)threadIdx.x < TK) write_rank_at(v, threadIdx.x, K, unit, sel_ids, sel_scores);
}

// Units of the fused interval selection hold at most this many candidates
// (summaries of up to 4,096 regions; topk_fused4_kernel below).
constexpr int FUSED_MAX_N = 16 * TK_WAVES * TK_PER;  // 4,096


// Appends the candidates whose key reaches t to sm.ids (and, with keys, the
// key to sm.keys), per wave in ballot order; misc[56] holds the count, zero
// on entry. Returns the total (a barrier comes first). Key k of thread tid is
// candidate j0 + tid + 1024 k; slots k >= nk are not looked at.
__device__ inline int compact_keys(const TkShared& sm, const uint32_t (&key)[TK_PER], uint32_t t,
                                   int64_t j0, bool keys, int nk = TK_PER) {
  const int tid = threadIdx.x, lane = tid & 63;
  unsigned long long msk[TK_PER];
  uint32_t wt = 0;
#pragma unroll
  for (int k = 0; k < TK_PER; ++k) {
    msk[k] = k < nk ? __ballot(key[k] >= t) : 0ull;  // nk: slots in use (block-uniform)
    wt += (uint32_t)__popcll(msk[k]);
  }
  uint32_t base = 0;
  if (lane == 0 && wt) base = atomicAdd(&sm.misc[56], wt);
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
  for (int k = 0; k < TK_PER; ++k) {
    if (msk[k]) {
      if (lane_in(msk[k])) {
        const uint32_t pos = base + lanes_below(msk[k]);
        sm.ids[pos] = (int32_t)(j0 + tid + TK_THREADS * k);
        if (keys) sm.keys[pos] = key[k];
      }
      base += (uint32_t)__popcll(msk[k]);
    }
  }
  __syncthreads();
  return (int)sm.misc[56];
}

// Exact scores of the survivors ids[0..M) of one (row, group) into keys[],
// on the fp64 matrix cores. qg: the row's query for the group as exact fp64
// [64 dims][4 heads]; Sg: the group's 64 bytes of candidate 0 (stride 256);
// wl: the weight of head 4g + (lane >> 4). A wave scores 16 survivors per
// chain of v_mfma_f64_4x4x4f64: the instruction's 4 blocks hold 4 survivors
// each and share the query, A[i][kk] = head i and B[kk][j] = survivor
// 16u + 4b + j (lane 16kk + 4b + i resp. j), step t of 16 taking dim
// 16kk + t, so each lane loads 16 contiguous bytes of one survivor. Every
// product and partial sum is exact in fp64; D[i][j] (lane 16i + 4b + j) then
// goes through group_score4's fp32 epilogue, heads summed in order. Waves
// take RS_Q groups of 16 at a time, groups wave, wave + 16, ... (3 fit the
// 64-register cap without spills). xb holds the query meanwhile (it is free
// until the sort).
constexpr int RS_Q = 3;
// qs: the query in LDS, [64 dims][4 heads] (a barrier since it was written)
__device__ inline void rescore_survivors_lds(const TkShared& sm, int M, const double* qs,
                                             const uint8_t* __restrict__ Sg, float wl, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int kk = lane >> 4, c16 = lane & 15, i = lane & 3;
  const int ngrp = (M + 15) >> 4;
  for (int u0 = wave; u0 < ngrp; u0 += RS_Q * TK_WAVES) {
    const int nq = min(RS_Q, (ngrp - u0 + TK_WAVES - 1) / TK_WAVES);  // groups u0 + 16q < ngrp
    uint4 bq[RS_Q];
#pragma unroll
    for (int q = 0; q < RS_Q; ++q) {
      const int m = min(16 * (u0 + TK_WAVES * q) + c16, M - 1);
      bq[q] = ldg16(Sg + (int64_t)sm.ids[m] * 256 + 16 * kk);
    }
    double acc[RS_Q];
#pragma unroll
    for (int q = 0; q < RS_Q; ++q) acc[q] = 0.0;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {  // dword t4 of the 16 bytes: steps 4 t4 .. 4 t4 + 3
      double qa[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) qa[e] = qs[(16 * kk + 4 * t4 + e) * 4 + i];
#pragma unroll
      for (int q = 0; q < RS_Q; ++q) {
        if (q >= nq) break;
        const uint32_t wd = t4 == 0 ? bq[q].x : t4 == 1 ? bq[q].y : t4 == 2 ? bq[q].z : bq[q].w;
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd, true);
        acc[q] = __builtin_amdgcn_mfma_f64_4x4x4f64(qa[0], (double)lo[0], acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f64_4x4x4f64(qa[1], (double)lo[1], acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f64_4x4x4f64(qa[2], (double)hi[0], acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f64_4x4x4f64(qa[3], (double)hi[1], acc[q], 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < RS_Q; ++q) {
      if (q >= nq) break;
      const float t = relu0((float)acc[q]) * wl;
      const float t1 = __shfl_down(t, 16, 64), t2 = __shfl_down(t, 32, 64),
                  t3 = __shfl_down(t, 48, 64);
      float sc = t + t1;
      sc = sc + t2;
      sc = sc + t3;
      const int m = 16 * (u0 + TK_WAVES * q) + lane;
      if (lane < 16 && m < M) sm.keys[m] = ord_key(sc);
    }
  }
  __syncthreads();
}
// qg: the row's e4m3 query for the group's 4 heads ([4 heads][64 dims]),
// staged in LDS as exact fp64 [64 dims][4 heads]
__device__ inline void rescore_survivors(const TkShared& sm, int M, const uint8_t* __restrict__ qg,
                                         const uint8_t* __restrict__ Sg, float wl, int tid) {
  double* qs = reinterpret_cast<double*>(sm.xb);
  if (tid < 256) qs[tid] = e4m3_f64(qg[(tid & 3) * 64 + (tid >> 2)]);
  __syncthreads();
  rescore_survivors_lds(sm, M, qs, Sg, wl, tid);
}

// One chunk of a (row, group)'s candidates: threshold, survivors, exact
// rescoring (intervals), exact selection. mode 0: the whole range, final
// output; mode 1: partial list, merged by the unit's last block.
// KIND: TK_EXACT reads exact scores from `bounds` (as float), TK_INTERVAL
// reads intervals (the fused interval selection is topk_fused4_kernel),
// TK_POOLED reads exact scores and the scorer's threshold keys (`pool`)
// and appends survivors to the unit's list (pool_select_tail; mode 2). The
// pooled path is its own instance so that the one-chunk kernel carries
// none of its code.
// Registers are capped for 8 waves per SIMD, so that two 1024-thread blocks
// share a CU when the chunk's LDS allows it (prefill-sized chunks of 4,096
// candidates): uncapped, the interval variant's scalar registers held it to
// one block per CU and 1.6x the time.
enum { TK_EXACT = 0, TK_INTERVAL = 1, TK_POOLED = 3 };

// Mode 2 (exact scores, a unit cut into chunks, the scorer's threshold keys
// at hand): the chunk's survivors sm.keys/ids[0..M) all reach a bound of the
// unit's 512th best, so the unit's best 512 lie among the union of every
// chunk's survivors, and among the best 512 of each chunk's. Each chunk
// appends those (at most 512) to the unit's list in `partial`, counted in
// arrivals[nunits + unit]; the last chunk to arrive sorts the list and
// writes the unit's selection. (The arrival counters are zeroed by the
// scorer of the same call.)
__device__ void pool_select_tail(const TkShared& sm, int M, int64_t unit, int nchunks,
                                 int64_t ncand, unsigned long long* __restrict__ partial,
                                 unsigned* __restrict__ arrivals, int64_t nunits,
                                 int32_t* __restrict__ sel_ids, float* __restrict__ sel_scores) {
  const int tid = threadIdx.x;
  unsigned long long v = 0ull;
  const int Mo = M < TK ? M : TK;
  if (M <= TK) {
    v = tid < M ? compose(sm.keys[tid], sm.ids[tid]) : 0ull;
  } else if (M <= TK_SORT) {
    v = sort_desc<TK_SORT>(tid < M ? compose(sm.keys[tid], sm.ids[tid]) : 0ull, sm);
  } else {
    collect_best(sm, M, TK);
    v = tid < TK ? sm.out[tid] : 0ull;
  }
  unsigned* const cnt = arrivals + nunits + unit;
  unsigned long long* const list = partial + unit * (int64_t)nchunks * TK;
  __shared__ unsigned sh_base;
  __shared__ int sh_last;
  if (tid == 0) sh_base = Mo ? atomicAdd(cnt, (unsigned)Mo) : 0u;
  __syncthreads();
  // device-scope stores (written through to where every die sees them), each
  // thread waits for its own, then one arrival per chunk: no release fence,
  // which would write back the die's whole L2 once per chunk
  if (tid < Mo)
    __hip_atomic_store(&list[sh_base + tid], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    sh_last = __hip_atomic_fetch_add(&arrivals[unit], 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == (unsigned)nchunks - 1u;
  __syncthreads();
  if (!sh_last) return;
  // every chunk's part is in (read with device-scope loads, which miss the
  // die's own cache): L >= the unit's K entries, all distinct
  const int L = (int)__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int K = ncand < TK ? (int)ncand : TK;
  auto ld = [&](int i) {
    return __hip_atomic_load(&list[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  unsigned long long w;
  if (L <= TK) {
    w = sort_desc<TK>(tid < L ? ld(tid) : 0ull, sm);
  } else if (L <= TK_SORT) {
    w = sort_desc<TK_SORT>(tid < L ? ld(tid) : 0ull, sm);
  } else {
    for (int i = tid; i < L; i += TK_THREADS) {
      const unsigned long long c = ld(i);
      sm.keys[i] = (uint32_t)(c >> 32);
      sm.ids[i] = (int32_t)~(uint32_t)c;
    }
    __syncthreads();
    collect_best(sm, L, K);
    w = sort_desc<TK>(tid < K ? sm.out[tid] : 0ull, sm);
  }
  write_rank(w, K, unit, sel_ids, sel_scores);
}

template <int KIND>
__global__ __launch_bounds__(TK_THREADS) __attribute__((amdgpu_waves_per_eu(8, 8))) void topk_chunk_kernel(
    int mode, const float2* __restrict__ bounds, int64_t R_cap,
    const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos, int64_t B,
    int64_t pos_limit, const uint8_t* __restrict__ q8, int64_t qs8, const float* __restrict__ w_head,
    int64_t w_stride, const uint8_t* __restrict__ S, int64_t ssb, int64_t chunk, int nchunks,
    unsigned long long* __restrict__ partial, const uint32_t* __restrict__ pool,
    unsigned* __restrict__ arrivals, int32_t* __restrict__ sel_ids,
    float* __restrict__ sel_scores, int64_t nunits, AppendArgs ap) {
  constexpr bool POOLED = KIND == TK_POOLED;
  constexpr bool EXACT = KIND == TK_EXACT || POOLED;
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int64_t)blockIdx.x >= nunits) {
    // workgroups past the units: the cache append of one decode row each
    // (first column of chunks only), on CUs the selection leaves idle
    if (blockIdx.y == 0)
      append_row_block(ap, (int64_t)blockIdx.x - nunits, reinterpret_cast<uint4(*)[32]>(smem),
                       reinterpret_cast<float4(*)[32][4]>(smem + 8 * 32 * 16));
    return;
  }
  const int64_t unit = blockIdx.x;
  const int c = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // mode 2 gathers up to nchunks x 512 survivors in the last block's LDS
  const TkShared sm =
      carve(smem, (int)(POOLED && (int64_t)nchunks * TK > chunk ? (int64_t)nchunks * TK : chunk));
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  const int64_t j0 = (int64_t)c * chunk;
  // keys of candidates tid + 1024 k in registers. The
  // chunk's slots of the score buffer are read before the row's candidate
  // count is known (it only masks them), all loads in flight at once; a lane
  // past the chunk's end reads its last slot again.
  float2 raw[TK_PER];
  int32_t seq;
  int64_t ncand;
  int N = 0;
  // the thread's keys (absent candidates 0) and its 4 group maxima
  uint32_t kh[TK_PER];
  uint32_t mx[4] = {0u, 0u, 0u, 0u};
  // mode 2: maxima of the unit's threshold keys from the scorer, entries
  // tid + 1024 (s + 4 i) in slot s
  uint32_t pv[4] = {0u, 0u, 0u, 0u};
  {
    const int nslot = (int)((R_cap - j0 < chunk) ? R_cap - j0 : chunk);
#pragma unroll
    for (int k = 0; k < TK_PER; ++k) {
      raw[k] = make_float2(0.f, 0.f);
      if (TK_THREADS * k < nslot) {
        const int i = min(tid + TK_THREADS * k, nslot - 1);
        if constexpr (EXACT) {
          const float s = reinterpret_cast<const float*>(bounds)[unit * R_cap + j0 + i];
          raw[k] = make_float2(s, s);
        } else {
          raw[k] = bounds[unit * R_cap + j0 + i];
        }
      }
    }
    // the unit's threshold keys, entry 64 wave + lane + 1024 (s + 4 i) in
    // slot s (coalesced; with at least 4,096 keys every wave gets as many)
    const int64_t npool = ((R_cap + 255) >> 8) * 8;
    const uint32_t* const pu = POOLED ? pool + unit * npool : nullptr;
    const int64_t pe0 = tid;
    if constexpr (POOLED) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t e = pe0 + TK_THREADS * s;
        if (e < npool) pv[s] = pu[e];
      }
    }
    unit_row(row_seq, row_pos, B, R_cap, pos_limit, row, &seq, &ncand);
    if (j0 < ncand) N = (int)((ncand - j0 < chunk) ? ncand - j0 : chunk);
    if constexpr (POOLED) {
      // keys of the first ceil(ncand / 32) entries were written by this call
      // (one per 32 candidates, 0 for those with none)
      const int64_t nvalid = (ncand + 31) >> 5;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (pe0 + TK_THREADS * s >= nvalid) pv[s] = 0u;
      for (int64_t e0 = pe0 + 4 * TK_THREADS; e0 < nvalid; e0 += 4 * TK_THREADS) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int64_t e = e0 + TK_THREADS * s;
          if (e < nvalid) pv[s] = pu[e] > pv[s] ? pu[e] : pv[s];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < TK_PER; ++k) {
      const bool have = tid + TK_THREADS * k < N;
      const uint32_t lo = have ? ord_key(raw[k].x) : 0u;
      kh[k] = EXACT ? lo : (have ? ord_key(raw[k].y) : 0u);
      mx[k & 3] = lo > mx[k & 3] ? lo : mx[k & 3];
    }
  }
  const int K = N < TK ? N : TK;
  // 1. tau = least over the waves of the wave's 32nd largest group maximum
  //    (at least 1: absent candidates, key 0, never survive). Mode 2 takes
  //    the same bound over the scorer's threshold keys instead: at least 512
  //    distinct candidates of the whole unit reach it (each slot a maximum
  //    over disjoint candidates), so the unit's 512th best does too.
  // (mode 2 takes the pool's bound alone: its chunks are small enough that
  // their own bound would be far below it)
  const uint32_t tw = wave_kth_largest4(POOLED ? pv : mx, TK / TK_WAVES);
  if (lane == 0) sm.misc[wave] = tw;
  if (tid == 0) sm.misc[56] = 0u;
  __syncthreads();
  uint32_t tau = 1u;
  {
    uint32_t t = sm.misc[0];
#pragma unroll
    for (int w = 1; w < TK_WAVES; ++w) t = min(t, sm.misc[w]);
    tau = t > 1u ? t : 1u;
  }
  // 2. survivors: upper key >= tau, appended per wave (their order is free:
  //    the selection sorts by (key, id))
  int M = compact_keys(sm, kh, tau, j0, EXACT,
                       POOLED ? (int)((chunk + TK_THREADS - 1) / TK_THREADS) : TK_PER);
  if constexpr (!EXACT) {
    if (M > TK_SORT) {
      // too many to sort directly: cut by T from the lower keys >= tau
      uint32_t kl[TK_PER];
#pragma unroll
      for (int k = 0; k < TK_PER; ++k) {
        kl[k] = tid + TK_THREADS * k < N ? ord_key(raw[k].x) : 0u;
      }
      if (tid == 0) sm.misc[56] = 0u;
      __syncthreads();
      M = compact_keys(sm, kl, tau, j0, true);
      const Boundary bd = radix_boundary(sm, M, K, 2);
      const uint32_t T = bd.P > 1u ? bd.P : 1u;
      if (tid == 0) sm.misc[56] = 0u;
      __syncthreads();
      M = compact_keys(sm, kh, T, j0, false);
    }
    // 3. exact scores of the survivors (matrix cores)
    const float wl = w_head[row * w_stride + 4 * g + (lane >> 4)];
    rescore_survivors(sm, M, q8 + row * qs8 + g * 256, S + (int64_t)seq * ssb + g * 64, wl, tid);
  }
  if constexpr (POOLED) {
    pool_select_tail(sm, M, unit, nchunks, ncand, partial, arrivals, nunits, sel_ids,
                     sel_scores);
    return;
  }
  // 4. exact best K of the survivors (M >= K), sorted: thread t < 512 gets rank t
  unsigned long long v;
  if (M <= TK) {
    v = sort_desc<TK>(tid < M ? compose(sm.keys[tid], sm.ids[tid]) : 0ull, sm);
  } else if (M <= TK_SORT) {
    v = sort_desc<TK_SORT>(tid < M ? compose(sm.keys[tid], sm.ids[tid]) : 0ull, sm);
  } else {
    collect_best(sm, M, K);
    v = sort_desc<TK>(tid < K ? sm.out[tid] : 0ull, sm);
  }
  if (mode == 0) write_rank(v, K, unit, sel_ids, sel_scores);
  else if (tid < TK) partial[(unit * nchunks + c) * TK + tid] = tid < K ? v : 0ull;
  if (mode == 0) return;
  // the unit's last block to arrive merges all chunk lists
  __shared__ int sh_last;
  if (!block_arrive_last(&arrivals[unit], (unsigned)nchunks, &sh_last)) return;
  merge_lists(partial + unit * (int64_t)nchunks * TK, nchunks, ncand, unit, smem, sel_ids,
              sel_scores);
}

// ---------------------------------------------------------------------------
// Fused intervals for four rows at once (prefill chunks): one workgroup per
// 4 consecutive rows and KV group g. When the rows share a sequence, the
// interval MFMA takes A = the 4 rows x the group's 4 heads (every MFMA row
// used) and B = 16 candidates, so each summary tile loaded serves all four
// rows; rows of different sequences get a pass each (A = one row's heads).
// Lane (n, qd) of the output then holds row qd's 4 head dots of candidate n
// and makes its interval. The intervals go to LDS as 16-bit key prefixes,
// rounded outward (lower key down to its prefix, upper key up to the
// prefix's last value), which keeps every bound below valid: the threshold
// is taken at 16-bit resolution anyway. Then: thresholds and survivors of
// the four units side by side, four waves each (16 candidates a thread);
// exact rescoring one unit after another by the whole workgroup (a unit
// with more than 1,024 survivors is redone here as in topk_chunk_kernel,
// cut and radix selected); the four sorts side by side, four waves each
// (one sort alone leaves a quarter of the block busy; four keep every
// SIMD at four waves). One workgroup per CU (64 KB of keys and 32 KB of
// composites beside the selection's LDS), so the register cap is that of
// 4 waves per SIMD.
// ---------------------------------------------------------------------------
constexpr int F4_KEYS = 4 * FUSED_MAX_N;  // u16 prefixes per array (4 rows)

// The bitonic network over 1,024 composites held four per thread by a group
// of 256 threads (four waves): element 4t + e in v[e], t the thread's index
// in the group. Partners one or two apart are in the thread, 4..255 apart in
// the wave (lane t ^ J/4, as above); the three stages with partners in
// another wave of the group go through xb, the group's 1,024 slots, in
// place (each thread writes its own four, a barrier, reads its partner's,
// a barrier). All groups of the block run it together (the barriers).
struct Bitonic4Ctx {
  int t;                   // the thread's index in its group
  int iw;                  // index of the wave's lane 0 in the group (wave-uniform)
  unsigned long long* xb;  // the group's 1,024 slots
};
template <int K, int J>
__device__ inline void bitonic4_stage(unsigned long long (&v)[4], const Bitonic4Ctx& c) {
  if constexpr (J < 4) {
    // elements e and e | J of the thread; descending where (i & K) == 0
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((e & J) != 0) continue;
      bool desc;
      if constexpr (K < 4) desc = (e & K) == 0;
      else desc = (c.t & (K >> 2)) == 0;
      const unsigned long long a = v[e], b = v[e | J];
      const bool keep = (a > b) == desc;  // the larger stays first where descending
      v[e] = keep ? a : b;
      v[e | J] = keep ? b : a;
    }
  } else if constexpr (J < 256) {
    constexpr int L = J >> 2;  // lane distance 1..32
    unsigned long long tm;     // lanes that keep the larger
    if constexpr ((K >> 2) < 64) tm = lanes_agree(L, K >> 2);
    else tm = ((c.iw & (K >> 2)) == 0) ? lanes_clear(L) : ~lanes_clear(L);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned long long p = ((unsigned long long)lane_xor<L>((uint32_t)(v[e] >> 32)) << 32) |
                                   lane_xor<L>((uint32_t)v[e]);
      v[e] = lane_in(~(__ballot(v[e] > p) ^ tm)) ? v[e] : p;
    }
  } else {
    constexpr int L = J >> 2;  // 64 or 128: another wave of the group
    ulonglong2* b = reinterpret_cast<ulonglong2*>(c.xb);
    b[2 * c.t] = make_ulonglong2(v[0], v[1]);
    b[2 * c.t + 1] = make_ulonglong2(v[2], v[3]);
    __syncthreads();
    const ulonglong2 p01 = b[2 * (c.t ^ L)], p23 = b[2 * (c.t ^ L) + 1];
    __syncthreads();
    const unsigned long long p[4] = {p01.x, p01.y, p23.x, p23.y};
    // wave-uniform: K / 4 and L are both at least 64
    const bool larger = ((c.t & (K >> 2)) == 0) == ((c.t & L) == 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = ((v[e] > p[e]) == larger) ? v[e] : p[e];
  }
}
template <int K, int J>
struct Bitonic4Merge {
  __device__ static inline void run(unsigned long long (&v)[4], const Bitonic4Ctx& c) {
    bitonic4_stage<K, J>(v, c);
    Bitonic4Merge<K, J / 2>::run(v, c);
  }
};
template <int K>
struct Bitonic4Merge<K, 0> {
  __device__ static inline void run(unsigned long long (&)[4], const Bitonic4Ctx&) {}
};
template <int K>
struct Bitonic4Sort {
  __device__ static inline void run(unsigned long long (&v)[4], const Bitonic4Ctx& c) {
    Bitonic4Sort<K / 2>::run(v, c);
    Bitonic4Merge<K, K / 2>::run(v, c);
  }
};
template <>
struct Bitonic4Sort<1> {
  __device__ static inline void run(unsigned long long (&)[4], const Bitonic4Ctx&) {}
};

// element i of a 4-array, i known only at run time (no dynamic indexing of
// a private array, which would go to scratch)
template <typename T>
__device__ inline T sel4(int i, T a, T b, T c, T d) {
  return i < 2 ? (i == 0 ? a : b) : (i == 2 ? c : d);
}

__global__ __launch_bounds__(TK_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) void
topk_fused4_kernel(const uint8_t* __restrict__ q8, int64_t qs8, int64_t R_cap,
                   const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos,
                   int64_t B, int64_t pos_limit, const float* __restrict__ w_head, int64_t w_stride,
                   const uint8_t* __restrict__ S, int64_t ssb, int32_t rows, int64_t nwg,
                   int32_t* __restrict__ sel_ids, float* __restrict__ sel_scores, AppendArgs ap) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int64_t)blockIdx.x >= nwg) {
    // workgroups past the units: the cache append of one decode row each
    append_row_block(ap, (int64_t)blockIdx.x - nwg, reinterpret_cast<uint4(*)[32]>(smem),
                     reinterpret_cast<float4(*)[32][4]>(smem + 8 * 32 * 16));
    return;
  }
  const int64_t r0 = (blockIdx.x >> 2) * 4;
  const int g = (int)(blockIdx.x & 3);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, qd = lane >> 4;
  const TkShared sm = carve(smem, FUSED_MAX_N);
  uint16_t* const kl16 = reinterpret_cast<uint16_t*>(smem + tk_smem_bytes(FUSED_MAX_N));
  uint16_t* const kh16 = kl16 + F4_KEYS;
  // the four units' composites for the final sort, [4][1,024]
  unsigned long long* const fin = reinterpret_cast<unsigned long long*>(kh16 + F4_KEYS);
  // the four rows (uniform): sequence (-1: no row / invalid) and candidates
  int32_t sq0, sq1, sq2, sq3;
  int64_t nc0, nc1, nc2, nc3;
  auto row_of = [&](int i, int32_t& si, int64_t& ni) {
    si = -1;
    ni = 0;
    if (r0 + i < rows) unit_row(row_seq, row_pos, B, R_cap, pos_limit, r0 + i, &si, &ni);
    if (ni > FUSED_MAX_N) ni = FUSED_MAX_N;  // (R_cap <= FUSED_MAX_N on this path)
  };
  row_of(0, sq0, nc0);
  row_of(1, sq1, nc1);
  row_of(2, sq2, nc2);
  row_of(3, sq3, nc3);
  auto SQ = [&](int i) { return sel4(i, sq0, sq1, sq2, sq3); };
  auto NC = [&](int i) { return sel4(i, nc0, nc1, nc2, nc3); };
  // the four units' exact queries for the rescoring (thread t: entry t % 256
  // of unit t / 256), loaded now and kept in LDS (sm.xb, [4][256]) once the
  // intervals are done, so that their latency hides behind the intervals
  const double qpre =
      NC(tid >> 8) > 0
          ? e4m3_f64(q8[(r0 + (tid >> 8)) * qs8 + g * 256 + (tid & 3) * 64 + ((tid & 255) >> 2)])
          : 0.0;
  int32_t s0 = -1;
  bool shared = true;
  int nmax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t si = SQ(i);
    const int64_t ni = NC(i);
    if (si < 0 || ni == 0) continue;
    if (s0 < 0) s0 = si;
    shared = shared && si == s0;
    nmax = max(nmax, (int)ni);
  }
  // this lane's output row qd: its weights and candidate count
  float w4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w4[i] = r0 + qd < rows ? w_head[(r0 + qd) * w_stride + 4 * g + i] : 0.f;
  // ---- intervals: one pass for rows sharing a sequence, else a pass per row
  const int npass = shared ? (s0 >= 0 ? 1 : 0) : 4;
  for (int ps = 0; ps < npass; ++ps) {
    const int prow = shared ? -1 : ps;  // the pass's row (per-row passes)
    const int32_t pseq = shared ? s0 : SQ(ps);
    const int pn = shared ? nmax : (int)NC(ps);
    if (pseq < 0 || pn == 0) continue;  // uniform
    // A: MFMA row n = 4 rl + h (shared) or h = n < 4 of the pass's row
    const int arow = shared ? (n >> 2) : prow;
    const int ah = shared ? (n & 3) : n;
    uint4 araw = make_uint4(0, 0, 0, 0);
    if (ah < 4 && SQ(arow) >= 0 && NC(arow) > 0)
      araw = ldg16(q8 + (r0 + arow) * qs8 + (4 * g + ah) * 64 + 16 * qd);
    const Bf16x16 aq = widen16(araw);
    // output row of this lane's D, and whether the lane holds one
    const int orow = shared ? qd : prow;
    const bool olane = shared || qd == 0;
    float wo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wo[i] = shared ? w4[i] : w_head[(r0 + prow) * w_stride + 4 * g + i];
    const int on = (int)NC(orow);
    const uint8_t* Sg = S + (int64_t)pseq * ssb + g * 64;
    const uint32_t jmax = (uint32_t)(pn - 1);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)Sg, (short)0, (int)((uint32_t)pn * 256u), RAW_RSRC3);
    // tile t of wave w: candidates 256 t + 16 w + n; 8 tiles per round trip
#pragma unroll 1
    for (int b = 0; b < FUSED_MAX_N / 256; b += 8) {
      if (256 * b >= pn) break;  // uniform
      uint4 bq[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t j = min((uint32_t)(256 * (b + u) + 16 * wave + n), jmax);
        bq[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rs, (int)(j * 256u + 16 * qd), 0, 0));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        f32x4 d, a;
        dot64(aq, widen16(bq[u]), d, a);
        const float2 iv = score_interval(d, a, wo);
        const int j = 256 * (b + u) + 16 * wave + n;
        if (olane && j < on) {
          kl16[orow * FUSED_MAX_N + j] = (uint16_t)(ord_key(iv.x) >> 16);
          kh16[orow * FUSED_MAX_N + j] = (uint16_t)(ord_key(iv.y) >> 16);
        }
      }
    }
  }
  __syncthreads();
  // ---- thresholds and survivors of the four units side by side, four waves
  //      (256 threads) each: thread t of unit ua's group holds candidates
  //      t + 256 k (k < 16), grouped by k % 4. tau = the least over the
  //      group's waves of the wave's 128th largest group maximum of the lower
  //      keys (at least 1): at least 512 distinct candidates reach it. The
  //      survivors (upper key >= tau) go to the unit's composite slots as
  //      ids (low words); misc[60 + ua] counts them (past 1,024 the unit is
  //      redone one unit at a time below).
  if (tid < 4) sm.misc[60 + tid] = 0u;
  reinterpret_cast<double*>(sm.xb)[tid] = qpre;
  __syncthreads();
  uint32_t* const fw = reinterpret_cast<uint32_t*>(fin);
  {
    const int ua = tid >> 8, t = tid & 255;
    const int Na = (int)NC(ua);
    uint32_t kha[16], mxa[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int j = t + 256 * k;
      const bool have = j < Na;
      const uint32_t lo = have ? (uint32_t)kl16[ua * FUSED_MAX_N + j] << 16 : 0u;
      kha[k] = have ? ((uint32_t)kh16[ua * FUSED_MAX_N + j] << 16) | 0xffffu : 0u;
      mxa[k & 3] = lo > mxa[k & 3] ? lo : mxa[k & 3];
    }
    const uint32_t twa = wave_kth_largest4(mxa, TK / 4);
    if (lane == 0) sm.misc[wave] = twa;
    __syncthreads();
    uint32_t taua;
    {
      const int w0 = 4 * ua;
      const uint32_t m =
          min(min(sm.misc[w0], sm.misc[w0 + 1]), min(sm.misc[w0 + 2], sm.misc[w0 + 3]));
      taua = m > 1u ? m : 1u;
    }
    unsigned long long msk[16];
    uint32_t wt = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      msk[k] = __ballot(kha[k] >= taua);
      wt += (uint32_t)__popcll(msk[k]);
    }
    uint32_t base = 0;
    if (lane == 0 && wt) base = atomicAdd(&sm.misc[60 + ua], wt);
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (msk[k]) {
        if (lane_in(msk[k])) {
          const uint32_t pos = base + lanes_below(msk[k]);
          if (pos < (uint32_t)TK_SORT) fw[2 * (ua * TK_SORT + pos)] = (uint32_t)(t + 256 * k);
        }
        base += (uint32_t)__popcll(msk[k]);
      }
    }
  }
  __syncthreads();
  const int Ma[4] = {(int)sm.misc[60], (int)sm.misc[61], (int)sm.misc[62], (int)sm.misc[63]};
  // ---- the four units' rescoring, one after another (a unit with more than
  //      1,024 survivors: its threshold, survivors and cut again here, the
  //      whole workgroup on it)
#pragma unroll 1
  for (int u = 0; u < 4; ++u) {
    const int64_t row = r0 + u;
    if (row >= rows) break;  // uniform
    const int N = (int)NC(u);
    const int32_t useq = SQ(u);
    const int K = N < TK ? N : TK;
    int M;
    const int Mu = sel4(u, Ma[0], Ma[1], Ma[2], Ma[3]);
    if (Mu <= TK_SORT) {
      M = Mu;
      if (tid < M) sm.ids[tid] = (int32_t)fw[2 * (u * TK_SORT + tid)];
      __syncthreads();
    } else {
    // keys of candidates tid + 1024 k (absent 0): lower prefix rounded down,
    // upper prefix rounded up to its last value
    uint32_t kh[TK_PER], mx[4];
#pragma unroll
    for (int k = 0; k < TK_PER; ++k) kh[k] = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = tid + TK_THREADS * k;
      const bool have = j < N;
      mx[k] = have ? (uint32_t)kl16[u * FUSED_MAX_N + j] << 16 : 0u;
      kh[k] = have ? ((uint32_t)kh16[u * FUSED_MAX_N + j] << 16) | 0xffffu : 0u;
    }
    // 1. tau: least over the waves of the wave's 32nd largest lower key
    const uint32_t tw = wave_kth_largest4(mx, TK / TK_WAVES);
    if (lane == 0) sm.misc[wave] = tw;
    if (tid == 0) sm.misc[56] = 0u;
    __syncthreads();
    uint32_t tau;
    {
      uint32_t t = sm.misc[0];
#pragma unroll
      for (int w = 1; w < TK_WAVES; ++w) t = min(t, sm.misc[w]);
      tau = t > 1u ? t : 1u;
    }
    // 2. survivors: upper key >= tau
    M = compact_keys(sm, kh, tau, 0, false, 4);
    if (M > TK_SORT) {
      // too many to sort directly: cut by T from the lower keys >= tau
      uint32_t kl[TK_PER];
#pragma unroll
      for (int k = 0; k < TK_PER; ++k) kl[k] = k < 4 ? mx[k] : 0u;
      if (tid == 0) sm.misc[56] = 0u;
      __syncthreads();
      M = compact_keys(sm, kl, tau, 0, true, 4);
      const Boundary bd = radix_boundary(sm, M, K, 2);
      const uint32_t T = bd.P > 1u ? bd.P : 1u;
      if (tid == 0) sm.misc[56] = 0u;
      __syncthreads();
      M = compact_keys(sm, kh, T, 0, false, 4);
    }
    }
    // 3. exact scores of the survivors (matrix cores)
    const float wl = w_head[row * w_stride + 4 * g + (lane >> 4)];
    if (M > 0)
      rescore_survivors_lds(sm, M, reinterpret_cast<const double*>(sm.xb) + 256 * u,
                            S + (int64_t)useq * ssb + g * 64, wl, tid);
    // 4. the unit's composites for the sort below: the survivors (at most
    //    1,024), or the best K of them when more survive (collect_best)
    unsigned long long* const fu = fin + u * TK_SORT;
    if (M <= TK_SORT) {
      fu[tid] = tid < M ? compose(sm.keys[tid], sm.ids[tid]) : 0ull;
    } else {
      collect_best(sm, M, K);
      fu[tid] = tid < K ? sm.out[tid] : 0ull;
    }
    __syncthreads();
  }
  // ---- the four units sorted at once, 256 threads (four waves) each,
  //      best first; thread t < 128 of a group writes ranks 4t .. 4t+3
  {
    const int us = tid >> 8, t = tid & 255;
    Bitonic4Ctx c;
    c.t = t;
    c.iw = __builtin_amdgcn_readfirstlane(t & ~63);
    c.xb = fin + us * TK_SORT;
    unsigned long long v[4];
    const ulonglong2* src = reinterpret_cast<const ulonglong2*>(c.xb);
    const ulonglong2 v01 = src[2 * t], v23 = src[2 * t + 1];
    v[0] = v01.x;
    v[1] = v01.y;
    v[2] = v23.x;
    v[3] = v23.y;
    Bitonic4Sort<TK_SORT>::run(v, c);
    const int64_t row = r0 + us;
    if (row < rows && t < TK / 4) {
      const int N = (int)NC(us);
      const int K = N < TK ? N : TK;
#pragma unroll
      for (int e = 0; e < 4; ++e) write_rank_at(v[e], 4 * t + e, K, row * 4 + g, sel_ids, sel_scores);
    }
  }
}

// Merge of the chunk lists of one (row, group): each list holds its chunk's
// exact best (at most 512) composites sorted best first, zero-padded, and
// composites are distinct. The best 512 of two such lists A, B are
// max(A[i], B[511 - i]), i < 512, a bitonic sequence, which the last nine
// bitonic stages sort. Lists are merged in pairs (two pairs at a time, one
// per half of the block) until one is left.
__device__ void merge_lists(const unsigned long long* __restrict__ src, int nchunks, int64_t ncand,
                            int64_t unit, unsigned char* smem, int32_t* __restrict__ sel_ids,
                            float* __restrict__ sel_scores) {
  unsigned long long* lists = reinterpret_cast<unsigned long long*>(smem);  // [nchunks][512]
  unsigned long long* xb = lists + (int64_t)nchunks * TK;                   // [2 groups][2][512]
  const int tid = threadIdx.x;
  const int grp = tid >> 9, i = tid & (TK - 1);
  for (int t = tid; t < nchunks * TK; t += TK_THREADS) lists[t] = src[t];
  __syncthreads();
  int nl = nchunks;
  BitonicCtx bc = bitonic_ctx(i, xb + grp * 2 * TK, TK, true);
  while (nl > 1) {
    const int npairs = nl >> 1;
    for (int p0 = 0; p0 < npairs; p0 += 2) {
      const int pr = p0 + grp;
      bc.active = pr < npairs;
      unsigned long long v = 0ull;
      if (bc.active) {
        const unsigned long long a = lists[(2 * pr) * TK + i];
        const unsigned long long b = lists[(2 * pr + 1) * TK + (TK - 1 - i)];
        v = a > b ? a : b;
      }
      v = BitonicMerge<TK, TK / 2>::run(v, bc);
      __syncthreads();
      if (bc.active) lists[pr * TK + i] = v;
      __syncthreads();
    }
    if (nl & 1) {
      // the odd list moves down to slot npairs (its old list is merged already)
      for (int t = tid; t < TK; t += TK_THREADS) lists[npairs * TK + t] = lists[(nl - 1) * TK + t];
      __syncthreads();
    }
    nl = npairs + (nl & 1);
  }
  const int K = ncand < TK ? (int)ncand : TK;
  if (tid < TK) write_rank(lists[tid], K, unit, sel_ids, sel_scores);
}

// chunks of at least this many candidates when a batch is cut further to
// fill the GPU
#ifndef S5_TOPK_MIN_CHUNK
#define S5_TOPK_MIN_CHUNK 16384
#endif

// exact scores over more than one chunk's worth of candidates: chunks of
// this many (more when 32 of them do not cover the summary), each keeping
// only what reaches the scorer's threshold bound
#ifndef S5_TOPK_POOL_CHUNK
#define S5_TOPK_POOL_CHUNK 4096
#endif

TopkPlan topk_plan(int32_t rows, int64_t R_cap) {
  if (score_exact_mode(rows) && R_cap > TK_MAX_N) {
    int64_t ch = S5_TOPK_POOL_CHUNK;
    if (ch * 32 < R_cap) ch = (R_cap + 31) / 32;
    ch = (ch + 63) / 64 * 64;
    TopkPlan p;
    p.chunk = ch;
    p.nchunks = (int32_t)((R_cap + ch - 1) / ch);
    return p;
  }
  // at most 16,384 candidates per chunk; a batch too small to fill the GPU
  // (rows * 4 units) is cut further, into chunks of at least
  // S5_TOPK_MIN_CHUNK, up to 16
  const int64_t units = (int64_t)rows * 4;
  const int64_t nmin = (R_cap + TK_MAX_N - 1) / TK_MAX_N;
  int64_t want = units > 0 ? (256 + units - 1) / units : 1;
  const int64_t by_size = (R_cap + S5_TOPK_MIN_CHUNK - 1) / S5_TOPK_MIN_CHUNK;
  if (want > by_size) want = by_size;
  if (want > 16) want = 16;
  int64_t n = want > nmin ? want : nmin;
  if (n < 1) n = 1;
  TopkPlan p;
  p.nchunks = (int32_t)n;
  int64_t ch = (R_cap + n - 1) / n;
  ch = (ch + 63) / 64 * 64;
  if (ch > TK_MAX_N) ch = TK_MAX_N;
  if (ch < 64) ch = 64;
  p.chunk = ch;
  return p;
}

size_t topk_partial_bytes(int32_t rows, int64_t R_cap) {
  const TopkPlan p = topk_plan(rows, R_cap);
  if (p.nchunks <= 1) return 0;
  return (size_t)rows * 4 * p.nchunks * TK * sizeof(unsigned long long);
}

size_t topk_pool_bytes(int32_t rows, int64_t R_cap) {
  if (!score_exact_mode(rows) || topk_plan(rows, R_cap).nchunks <= 1) return 0;
  return (size_t)rows * 4 * (size_t)((R_cap + 255) / 256) * 8 * sizeof(uint32_t);
}

// the append's LDS (z and e, e*k of 8 tokens x 32 lanes) fits in every
// selection launch's dynamic LDS
static_assert(8 * 32 * 16 + 8 * 32 * 64 <= TK * 8 + 2 * TK_SORT * 8, "append LDS");

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const unsigned units = (unsigned)a.rows * 4u;
  AppendArgs ap{};
  unsigned napp = 0;
  if (a.append) {
    ap = *a.append;
    napp = (unsigned)ap.rows;
  }
  if (a.fused) {
    const size_t sm = tk_smem_bytes(FUSED_MAX_N) + (size_t)2 * F4_KEYS * sizeof(uint16_t) +
                      (size_t)4 * TK_SORT * sizeof(unsigned long long);
    hipError_t e = hipFuncSetAttribute((const void*)topk_fused4_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    const int64_t nwg = ((int64_t)a.rows + 3) / 4 * 4;
    hipLaunchKernelGGL(topk_fused4_kernel, dim3((unsigned)(nwg + napp)), dim3(TK_THREADS), sm,
                       stream, a.q8, a.q8_stride_row, a.R_cap, a.row_seq, a.row_pos, a.B,
                       a.pos_limit, a.w_head, a.w_stride_row, a.summary, a.ssb, a.rows, nwg,
                       a.sel_ids, a.sel_scores, ap);
    return hipGetLastError();
  }
  const TopkPlan p = topk_plan(a.rows, a.R_cap);
  // mode 0: one chunk per unit; 1: chunk lists merged by the last chunk;
  // 2 (exact scores with the scorer's threshold keys): survivor lists
  const int mode = p.nchunks == 1 ? 0 : (a.exact && a.pool ? 2 : 1);
  size_t sm = tk_smem_bytes((int)p.chunk);
  if (mode == 1) {
    const size_t sm_merge = (size_t)(p.nchunks + 4) * TK * sizeof(unsigned long long);
    if (sm_merge > sm) sm = sm_merge;
  } else if (mode == 2 && (int64_t)p.nchunks * TK > p.chunk) {
    sm = tk_smem_bytes(p.nchunks * TK);
  }
  const void* fn = mode == 2  ? (const void*)topk_chunk_kernel<TK_POOLED>
                   : a.exact ? (const void*)topk_chunk_kernel<TK_EXACT>
                             : (const void*)topk_chunk_kernel<TK_INTERVAL>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const dim3 grid(units + napp, (unsigned)p.nchunks);
  if (mode == 2)
    hipLaunchKernelGGL(topk_chunk_kernel<TK_POOLED>, grid, dim3(TK_THREADS), sm, stream, mode,
                       a.bounds, a.R_cap, a.row_seq, a.row_pos, a.B,
                       a.pos_limit, a.q8, a.q8_stride_row, a.w_head, a.w_stride_row, a.summary,
                       a.ssb, p.chunk,
                       p.nchunks, a.partial, a.pool, a.arrivals, a.sel_ids, a.sel_scores,
                       (int64_t)units, ap);
  else if (a.exact)
    hipLaunchKernelGGL(topk_chunk_kernel<TK_EXACT>, grid, dim3(TK_THREADS), sm, stream, mode,
                       a.bounds, a.R_cap, a.row_seq, a.row_pos, a.B,
                       a.pos_limit, a.q8, a.q8_stride_row, a.w_head, a.w_stride_row, a.summary,
                       a.ssb, p.chunk,
                       p.nchunks, a.partial, nullptr, a.arrivals, a.sel_ids, a.sel_scores,
                       (int64_t)units, ap);
  else
    hipLaunchKernelGGL(topk_chunk_kernel<TK_INTERVAL>, grid, dim3(TK_THREADS), sm, stream, mode,
                       a.bounds, a.R_cap, a.row_seq, a.row_pos, a.B,
                       a.pos_limit, a.q8, a.q8_stride_row, a.w_head, a.w_stride_row, a.summary,
                       a.ssb, p.chunk,
                       p.nchunks, a.partial, nullptr, a.arrivals, a.sel_ids, a.sel_scores,
                       (int64_t)units, ap);
  return hipGetLastError();
}

}  // namespace s5
