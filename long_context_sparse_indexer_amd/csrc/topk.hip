// Top-512 region selection per (row, KV group).
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// keep the top 512 regions by (-score, id), ascending: best score first,
// equal scores by the smaller region id. Fewer than 512 candidates keep all.
//
// Input: the score kernel's exact score per candidate (few rows), which is
// selected from directly, or its interval [lo, hi] holding the exact score. Per (row, group) and chunk of candidates (one 1024-thread
// workgroup, everything in LDS; gfx950 gives a workgroup up to 160 KB), from
// intervals:
//   1. T = the top 22 bits of the K-th largest lower bound, the rest zero
//      (K = min(512, candidates)), so T <= that bound;
//   2. C = the candidates whose upper bound reaches T, kept in id order.
//      C holds every candidate of the exact top K: each of those has
//      hi >= exact score >= K-th largest exact score >= K-th largest lo >= T;
//   3. every member of C is rescored exactly (exact.hpp);
//   4. the best K of C by (-exact score, id) are selected and sorted.
// Candidate ranges past 16,384, and batches too small to fill the GPU, are
// cut into chunks: each chunk keeps its exact best 512, sorted; the last
// chunk of a (row, group) to finish (an arrival counter per unit, zeroed by
// the query prep of the same call) merges the chunk lists pairwise.
//
// Selecting the best K of N exact keys (scores mapped to 32-bit keys that
// order like the scores, -0 taken as +0; ties broken by id):
//   radix select in 3 passes (11, 11, 10 bits) finds the boundary: a key
//   prefix P under a mask, such that keys above P are all taken and `need`
//   keys with prefix P are taken in list order (list order is id order); the
//   passes stop early when the boundary bin is taken whole. The bins are
//   scanned by all threads at once (two bins each, a block-wide scan). The
//   selected elements are then sorted by a bitonic network.
#include "device.hpp"
#include "exact.hpp"
#include "launch.hpp"

namespace s5 {

constexpr int TK = 512;
constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int64_t TK_MAX_N = 16384;
constexpr int TK_MAX_CHUNKS = 32;
constexpr int TK_BINS = 2048;

__device__ inline uint32_t ord_key(float s) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
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
};

__host__ __device__ inline size_t tk_smem_bytes(int nmax) {
  return (size_t)TK * 8 + (size_t)(TK_BINS + 64) * 4 + (size_t)nmax * 8;
}

__device__ inline TkShared carve(unsigned char* base, int nmax) {
  TkShared s;
  s.out = reinterpret_cast<unsigned long long*>(base);
  s.hist = reinterpret_cast<uint32_t*>(base + TK * 8);
  s.misc = s.hist + TK_BINS;
  s.keys = s.misc + 64;
  s.ids = reinterpret_cast<int32_t*>(s.keys + nmax);
  return s;
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
};

// Radix select over keys[0..N), 1 <= K <= N: keys with (k & mask) > P are
// the K - need best; `need` more come from the keys with (k & mask) == P.
// With early = false and passes = 3 all 32 bits are resolved (P is then the
// K-th best key); fewer passes leave P = the K-th best key's top bits.
__device__ Boundary radix_boundary(const TkShared& sm, int N, int K, bool early, int passes = 3) {
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
    if (early && need == cnt) break;
  }
  Boundary bd;
  bd.P = P;
  bd.mask = mask;
  bd.need = need;
  return bd;
}

__device__ void collect_best(const TkShared& sm, int N, int K, const int32_t* ids, int32_t id_base);
__device__ void rank_sort(const TkShared& sm, int K);

// Best K of keys[0..N) (ids[i], or id_base + i when ids is null) as sorted
// composites: sm.out[rank] for rank < K; sm.out[K..TK) = 0. Requires N >= K.
__device__ void select_sorted(const TkShared& sm, int N, int K, const int32_t* ids,
                              int32_t id_base) {
  const int tid = threadIdx.x;
  if (N == K) {
    // everything is taken
    for (int i = tid; i < K; i += TK_THREADS) sm.out[i] = compose(sm.keys[i], ids ? ids[i] : id_base + i);
    __syncthreads();
  } else {
    collect_best(sm, N, K, ids, id_base);
  }
  rank_sort(sm, K);
}

// keys[0..N) -> sm.out[0..K): the best K (any order), N > K >= 1 or K == 0
__device__ void collect_best(const TkShared& sm, int N, int K, const int32_t* ids,
                             int32_t id_base) {
  const int tid = threadIdx.x;
  Boundary bd = {0u, 0u, 0u};
  if (K > 0) bd = radix_boundary(sm, N, K, true);
  const int seg = (N + TK_THREADS - 1) / TK_THREADS;
  const int i0 = min(N, tid * seg), i1 = min(N, i0 + seg);
  uint32_t ngt = 0, neq = 0;
  if (K > 0)
    for (int i = i0; i < i1; ++i) {
      const uint32_t m = sm.keys[i] & bd.mask;
      ngt += m > bd.P;
      neq += m == bd.P;
    }
  uint32_t tot;
  uint32_t gt_off = block_excl_scan(ngt, sm.misc, &tot);
  uint32_t eq_off = block_excl_scan(neq, sm.misc, &tot);
  const uint32_t eq_base = (uint32_t)K - bd.need;
  if (K > 0)
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = sm.keys[i];
      const uint32_t m = k & bd.mask;
      if (m < bd.P) continue;
      const int32_t id = ids ? ids[i] : id_base + i;
      if (m > bd.P) {
        sm.out[gt_off++] = compose(k, id);
      } else {
        if (eq_off < bd.need) sm.out[eq_base + eq_off] = compose(k, id);
        ++eq_off;
      }
    }
  __syncthreads();
}

// Bitonic network on 512 composites held one per thread by a group of 512
// threads (i = index in the group; groups are whole waves). Stage (k, j):
// compare with element i ^ j, keep the larger where the k-block runs
// descending and i is the lower index of the pair (or neither), else the
// smaller. Partners closer than 64 are in the wave (DPP or a lane permute);
// farther ones go through xb (the group's 2 x 512 slots, alternated so one
// barrier per stage suffices). Every thread of the block runs the stages
// (the barriers); inactive ones exchange nothing.
struct BitonicCtx {
  int i, lane;
  unsigned long long* xb;
  bool active;
  int flip;
};

template <int K, int J>
__device__ inline unsigned long long bitonic_stage(unsigned long long v, BitonicCtx& c) {
  unsigned long long p;
  if constexpr (J >= 64) {
    unsigned long long* b = c.xb + 512 * c.flip;
    c.flip ^= 1;
    if (c.active) b[c.i] = v;
    __syncthreads();
    p = c.active ? b[c.i ^ J] : 0ull;
  } else {
    p = lane_xor64<J>(v, c.lane);
  }
  const bool desc = (c.i & K) == 0;
  const bool lower = (c.i & J) == 0;
  return (desc == lower) ? (v > p ? v : p) : (v < p ? v : p);
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

// sm.out[0..K) (distinct composites, any order) -> sorted best first;
// sm.out[K..TK) = 0. Threads 0..511 sort, with the histogram as exchange space.
__device__ void rank_sort(const TkShared& sm, int K) {
  const int tid = threadIdx.x;
  BitonicCtx c;
  c.i = tid & (TK - 1);
  c.lane = tid & 63;
  c.active = tid < TK;
  c.xb = reinterpret_cast<unsigned long long*>(sm.hist);  // 2 x 512 slots
  c.flip = 0;
  unsigned long long v = (c.active && c.i < K) ? sm.out[c.i] : 0ull;
  v = BitonicSort<TK>::run(v, c);
  __syncthreads();
  if (c.active) sm.out[c.i] = v;
  __syncthreads();
}

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

__device__ inline void write_final(const TkShared& sm, int K, int64_t unit, int32_t* sel_ids,
                                   float* sel_scores) {
  for (int i = threadIdx.x; i < TK; i += TK_THREADS) {
    const unsigned long long c = sm.out[i];
    const bool have = i < K;
    sel_ids[unit * TK + i] = have ? (int32_t)(~(uint32_t)c) : -1;
    if (sel_scores) sel_scores[unit * TK + i] = have ? key_score((uint32_t)(c >> 32)) : 0.0f;
  }
}

// One chunk of a (row, group)'s candidates: interval filter, exact rescoring,
// exact selection. mode 0: the whole range, final output; mode 1: partial list.
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(
    int mode, int exact, const float2* __restrict__ bounds, int64_t R_cap, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, int64_t B, int64_t pos_limit,
    const double* __restrict__ q64, const float* __restrict__ w_head, int64_t w_stride,
    const uint8_t* __restrict__ S, int64_t ssb, int64_t chunk, int nchunks,
    unsigned long long* __restrict__ partial, unsigned* __restrict__ arrivals,
    int32_t* __restrict__ sel_ids, float* __restrict__ sel_scores) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t unit = blockIdx.x;
  const int c = blockIdx.y;
  const int tid = threadIdx.x;
  const TkShared sm = carve(smem, (int)chunk);
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  int32_t seq;
  int64_t ncand;
  unit_row(row_seq, row_pos, B, R_cap, pos_limit, row, &seq, &ncand);
  const int64_t j0 = (int64_t)c * chunk;
  int N = 0;
  if (j0 < ncand) N = (int)((ncand - j0 < chunk) ? ncand - j0 : chunk);
  const int K = N < TK ? N : TK;
  const float2* bsrc = bounds + unit * R_cap + j0;
  int M = 0;
  const int32_t* sel_from = sm.ids;  // ids of keys[0..M), or j0 + index when exact
  int32_t id_base = 0;
  if (exact) {
    // exact scores: select straight from them
    const float* ssrc = reinterpret_cast<const float*>(bounds) + unit * R_cap + j0;
    for (int i = tid; i < N; i += TK_THREADS) sm.keys[i] = ord_key(ssrc[i]);
    __syncthreads();
    M = N;
    sel_from = nullptr;
    id_base = (int32_t)j0;
  } else if (K > 0) {
    // 1. K-th largest lower bound (upper bounds parked in ids[] meanwhile)
    for (int i = tid; i < N; i += TK_THREADS) {
      const float2 b = bsrc[i];
      sm.keys[i] = ord_key(b.x);
      sm.ids[i] = (int32_t)ord_key(b.y);
    }
    __syncthreads();
    // two passes fix the top 22 bits of the K-th largest lower bound; T (those
    // bits, the rest zero) is at most that bound, which is all the filter needs
    const Boundary bd = radix_boundary(sm, N, K, false, 2);
    const uint32_t T = bd.P;
    // 2. candidates whose upper bound reaches T, in id order: each thread
    //    takes its segment's upper bounds into registers, the scan orders the
    //    writes (its barriers separate every read from every write)
    const int seg = (N + TK_THREADS - 1) / TK_THREADS;  // <= TK_MAX_N / TK_THREADS
    const int i0 = min(N, tid * seg), i1 = min(N, i0 + seg);
    uint32_t flags = 0, cnt = 0;
#pragma unroll
    for (int k = 0; k < (int)(TK_MAX_N / TK_THREADS); ++k) {
      const int i = i0 + k;
      if (i < i1 && (uint32_t)sm.ids[i] >= T) {
        flags |= 1u << k;
        ++cnt;
      }
    }
    uint32_t total;
    uint32_t off = block_excl_scan(cnt, sm.misc, &total);
#pragma unroll
    for (int k = 0; k < (int)(TK_MAX_N / TK_THREADS); ++k)
      if ((flags >> k) & 1u) sm.ids[off++] = (int32_t)(j0 + i0 + k);
    M = (int)total;
    __syncthreads();
    // 3. exact scores of the survivors: two threads per candidate (dims
    //    0..31 and 32..63); partial fp64 sums are exact, so is their sum
    double* q_lds = reinterpret_cast<double*>(sm.hist);  // 256 doubles (the histogram is free now)
    const double* qg = q64 + (row * 4 + g) * 256;
    for (int i = tid; i < 256; i += TK_THREADS) q_lds[i] = qg[i];
    __syncthreads();
    const uint8_t* Sg = S + (int64_t)seq * ssb + g * 64;
    float w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w4[i] = w_head[row * w_stride + 4 * g + i];
    const int half = tid & 1;
    for (int m0 = 0; m0 < M; m0 += TK_THREADS / 2) {
      const int m = m0 + (tid >> 1);
      double a[4] = {0.0, 0.0, 0.0, 0.0};
      if (m < M) exact_half_dots(Sg + (int64_t)sm.ids[m] * 256 + 32 * half, q_lds + 128 * half, a);
#pragma unroll
      for (int h = 0; h < 4; ++h) a[h] += __shfl_xor(a[h], 1, 64);
      if (m < M && half == 0) sm.keys[m] = ord_key(group_score4((float)a[0], (float)a[1], (float)a[2], (float)a[3], w4));
    }
    __syncthreads();
  }
  // 4. exact best K of the survivors
  if (mode == 0) {
    select_sorted(sm, M, K, sel_from, id_base);
    write_final(sm, K, unit, sel_ids, sel_scores);
    return;
  }
  // chunk list out: its best K, sorted, zero-padded to 512; the unit's last
  // block to arrive merges all of them
  select_sorted(sm, M, K, sel_from, id_base);
  unsigned long long* dst = partial + (unit * nchunks + c) * TK;
  for (int i = tid; i < TK; i += TK_THREADS) dst[i] = sm.out[i];
  __shared__ int sh_last;
  if (!block_arrive_last(&arrivals[unit], (unsigned)nchunks, &sh_last)) return;
  merge_lists(partial + unit * (int64_t)nchunks * TK, nchunks, ncand, unit, smem, sel_ids,
              sel_scores);
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
  BitonicCtx bc;
  bc.i = i;
  bc.lane = tid & 63;
  bc.xb = xb + grp * 2 * TK;
  bc.flip = 0;
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
  for (int t = tid; t < TK; t += TK_THREADS) {
    const unsigned long long c = lists[t];
    const bool have = t < K;
    sel_ids[unit * TK + t] = have ? (int32_t)(~(uint32_t)c) : -1;
    if (sel_scores) sel_scores[unit * TK + t] = have ? key_score((uint32_t)(c >> 32)) : 0.0f;
  }
}

TopkPlan topk_plan(int32_t rows, int64_t R_cap) {
  // at most 16,384 candidates per chunk; a batch too small to fill the GPU
  // (rows * 4 units) is cut further, into chunks of at least 2,048, up to 16
  const int64_t units = (int64_t)rows * 4;
  const int64_t nmin = (R_cap + TK_MAX_N - 1) / TK_MAX_N;
  int64_t want = units > 0 ? (256 + units - 1) / units : 1;
  const int64_t by_size = (R_cap + 2047) / 2048;
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

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const TopkPlan p = topk_plan(a.rows, a.R_cap);
  const unsigned units = (unsigned)a.rows * 4u;
  size_t sm = tk_smem_bytes((int)p.chunk);
  const size_t sm_merge = (size_t)(p.nchunks + 4) * TK * sizeof(unsigned long long);
  if (p.nchunks > 1 && sm_merge > sm) sm = sm_merge;
  hipError_t e = hipFuncSetAttribute((const void*)topk_chunk_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const int mode = p.nchunks == 1 ? 0 : 1;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(units, (unsigned)p.nchunks), dim3(TK_THREADS), sm,
                     stream, mode, a.exact ? 1 : 0, a.bounds, a.R_cap, a.row_seq, a.row_pos, a.B, a.pos_limit,
                     a.q64, a.w_head, a.w_stride_row, a.summary, a.ssb, p.chunk, p.nchunks,
                     a.partial, a.arrivals, a.sel_ids, a.sel_scores);
  return hipGetLastError();
}

}  // namespace s5
