// Top-512 region selection per (row, KV group).
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// keep the top 512 regions by (-score, id), ascending: best score first,
// equal scores by the smaller region id. Fewer than 512 candidates keep all.
//
// Input: the score kernel's interval [lo, hi] per candidate, which holds the
// exact score. Per (row, group) and chunk of candidates (one 1024-thread
// workgroup, everything in LDS; gfx950 gives a workgroup up to 160 KB):
//   1. T = the K-th largest lower bound (K = min(512, candidates));
//   2. C = the candidates whose upper bound reaches T, kept in id order.
//      C holds every candidate of the exact top K: each of those has
//      hi >= exact score >= K-th largest exact score >= K-th largest lo = T;
//   3. every member of C is rescored exactly (exact.hpp);
//   4. the best K of C by (-exact score, id) are selected and sorted.
// Candidate ranges past 16,384, and batches too small to fill the GPU, are
// cut into chunks: each chunk keeps its exact best 512 in order; the last
// chunk of a (row, group) to finish (an arrival counter per unit, zeroed by
// the query prep of the same call) ranks the elements of the chunk lists
// against each other.
//
// Selecting the best K of N exact keys (scores mapped to 32-bit keys that
// order like the scores, -0 taken as +0; ties broken by id):
//   radix select in 3 passes (11, 11, 10 bits) finds the boundary: a key
//   prefix P under a mask, such that keys above P are all taken and `need`
//   keys with prefix P are taken in list order (list order is id order); the
//   passes stop early when the boundary bin is taken whole. The bins are
//   scanned by all threads at once (two bins each, a block-wide scan). Then
//   every selected element gets its rank by counting the selected elements
//   above it, which sorts them without a sorting network.
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
  uint32_t* rank;           // [TK]
};

__host__ __device__ inline size_t tk_smem_bytes(int nmax) {
  return (size_t)TK * 8 + (size_t)TK * 4 + (size_t)(TK_BINS + 64) * 4 + (size_t)nmax * 8;
}

__device__ inline TkShared carve(unsigned char* base, int nmax) {
  TkShared s;
  s.out = reinterpret_cast<unsigned long long*>(base);
  s.rank = reinterpret_cast<uint32_t*>(base + TK * 8);
  s.hist = s.rank + TK;
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
// With early = false all 32 bits are resolved (P is then the K-th best key).
__device__ Boundary radix_boundary(const TkShared& sm, int N, int K, bool early) {
  const int tid = threadIdx.x;
  uint32_t P = 0, mask = 0, need = (uint32_t)K;
  const int shifts[3] = {21, 10, 0};
  const int bits[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
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

// sm.out[0..K) (distinct composites, any order) -> sorted best first;
// sm.out[K..TK) = 0
__device__ void rank_sort(const TkShared& sm, int K) {
  const int tid = threadIdx.x;
  // rank of each selected composite (all distinct): two threads per element,
  // each counting half of the list; 16-byte LDS reads, eight in flight
  const int e = tid & (TK - 1), half = tid >> 9;
  uint32_t r = 0;
  unsigned long long mine = 0;
  if (e < K) {
    mine = sm.out[e];
    const int j0 = half * (TK / 2);
    const int j1 = min(K, j0 + TK / 2);
    const ulonglong2* o2 = reinterpret_cast<const ulonglong2*>(sm.out);
    int j = j0;
    for (; j + 16 <= j1; j += 16) {
      ulonglong2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = o2[(j >> 1) + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += (v[u].x > mine) + (v[u].y > mine);
    }
    for (; j < j1; ++j) r += sm.out[j] > mine;
  }
  if (half == 1) sm.rank[e] = r;
  __syncthreads();
  if (half == 0 && e < K) r += sm.rank[e];
  __syncthreads();
  if (half == 0 && e < K) sm.out[r] = mine;  // distinct ranks: a permutation of 0..K-1
  if (half == 1 && K + e < TK) sm.out[K + e] = 0ull;
  __syncthreads();
}

__device__ void merge_lists(const unsigned long long* __restrict__ src, int nchunks, int K,
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
    int mode, const float2* __restrict__ bounds, int64_t R_cap, const int32_t* __restrict__ row_seq,
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
  if (K > 0) {
    // 1. K-th largest lower bound (upper bounds parked in ids[] meanwhile)
    for (int i = tid; i < N; i += TK_THREADS) {
      const float2 b = bsrc[i];
      sm.keys[i] = ord_key(b.x);
      sm.ids[i] = (int32_t)ord_key(b.y);
    }
    __syncthreads();
    const Boundary bd = radix_boundary(sm, N, K, false);
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
  select_sorted(sm, M, K, sm.ids, 0);
  if (mode == 0) {
    write_final(sm, K, unit, sel_ids, sel_scores);
    return;
  }
  // chunk list out; the unit's last block to arrive merges all of them
  unsigned long long* dst = partial + (unit * nchunks + c) * TK;
  for (int i = tid; i < TK; i += TK_THREADS) dst[i] = sm.out[i];
  __shared__ int sh_last;
  __syncthreads();  // every thread's list stores have completed
  if (tid == 0) {
    __threadfence();  // release: the block's stores become visible device-wide
    sh_last = atomicAdd(&arrivals[unit], 1u) == (unsigned)(nchunks - 1);
    if (sh_last) __threadfence();  // acquire: drop stale copies before reading the lists
  }
  __syncthreads();
  if (!sh_last) return;
  const int Kall = ncand < TK ? (int)ncand : TK;
  merge_lists(partial + unit * (int64_t)nchunks * TK, nchunks, Kall, unit, smem, sel_ids,
              sel_scores);
}

// Merge of the chunk lists of one (row, group): each list is sorted best
// first and composites are distinct, so an element's rank in the union is its
// index in its own list plus, for every other list, the number of elements
// above it there (a binary search). Elements ranked below K go to their rank:
// the output is sorted. smem holds (nchunks + 1) * TK composites.
__device__ void merge_lists(const unsigned long long* __restrict__ src, int nchunks, int K,
                            int64_t unit, unsigned char* smem, int32_t* __restrict__ sel_ids,
                            float* __restrict__ sel_scores) {
  unsigned long long* lists = reinterpret_cast<unsigned long long*>(smem);  // [nchunks][TK]
  unsigned long long* outl = lists + (int64_t)nchunks * TK;                 // [TK]
  const int N = nchunks * TK;
  for (int i = threadIdx.x; i < N; i += TK_THREADS) lists[i] = src[i];
  for (int i = threadIdx.x; i < TK; i += TK_THREADS) outl[i] = 0ull;
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += TK_THREADS) {
    const unsigned long long x = lists[i];
    if (x == 0ull) continue;  // padding
    const int c = i / TK;
    int rank = i - c * TK;
    for (int o = 0; o < nchunks && rank < K; ++o) {
      if (o == c) continue;
      const unsigned long long* L = lists + (int64_t)o * TK;
      int lo = 0, hi = TK;  // count of L[j] > x: L is descending
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (L[mid] > x) lo = mid + 1; else hi = mid;
      }
      rank += lo;
    }
    if (rank < K) outl[rank] = x;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < TK; i += TK_THREADS) {
    const unsigned long long c = outl[i];
    const bool have = i < K;
    sel_ids[unit * TK + i] = have ? (int32_t)(~(uint32_t)c) : -1;
    if (sel_scores) sel_scores[unit * TK + i] = have ? key_score((uint32_t)(c >> 32)) : 0.0f;
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
  const size_t sm_merge = (size_t)(p.nchunks + 1) * TK * sizeof(unsigned long long);
  if (p.nchunks > 1 && sm_merge > sm) sm = sm_merge;
  hipError_t e = hipFuncSetAttribute((const void*)topk_chunk_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const int mode = p.nchunks == 1 ? 0 : 1;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(units, (unsigned)p.nchunks), dim3(TK_THREADS), sm,
                     stream, mode, a.bounds, a.R_cap, a.row_seq, a.row_pos, a.B, a.pos_limit,
                     a.q64, a.w_head, a.w_stride_row, a.summary, a.ssb, p.chunk, p.nchunks,
                     a.partial, a.arrivals, a.sel_ids, a.sel_scores);
  return hipGetLastError();
}

}  // namespace s5
