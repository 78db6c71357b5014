// Top-512 region selection per (row, KV group).
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"), indexer commit note:
// keep the top 512 regions by (-score, id), ascending: best score first,
// equal scores by the smaller region id. Fewer than 512 candidates keep all.
//
// Scores map to 32-bit keys that order like the scores (-0 taken as +0);
// ties are then broken by id. Selection of the best K of N keys held in LDS:
//   1. radix select, 4 passes of 8 bits from the top, finds the K-th best key
//      T and how many keys equal to T are needed (histograms per wave in LDS,
//      a suffix scan over the 256 bins);
//   2. every key > T is taken, and the first `need` keys == T in list order;
//      the lists are built so that list order is id order among equal keys;
//   3. a bitonic sort of the K composites (key << 32 | ~id) gives the final
//      (-score, id) order.
// One workgroup (1024 threads) owns one list of up to 16,384 keys in LDS
// (gfx950 gives a workgroup up to 160 KB). Longer candidate ranges, or batches
// too small to fill the GPU, are cut into chunks: each chunk keeps its best
// 512 in order, and a merge pass selects from the chunk lists laid end to end
// (chunk order is id order, so equal keys stay in id order).
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

constexpr int TK = 512;
constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int64_t TK_MAX_N = 16384;
constexpr int TK_MAX_CHUNKS = 32;

__device__ inline uint32_t ord_key(float s) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_score(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}

struct TkShared {
  uint32_t* keys;   // [nmax]
  int32_t* ids;     // [nmax] or null (ids = base + position)
  uint32_t* hist;   // [TK_WAVES * 256]
  uint32_t* suf;    // [256]
  uint32_t* scan;   // [64]
  unsigned long long* out;  // [TK]
};

// exclusive scan of v over the 1024 threads; *total gets the sum
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* scan, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) scan[wave] = x;
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t t = scan[w];
      scan[32 + w] = acc;
      acc += t;
    }
    scan[63] = acc;
  }
  __syncthreads();
  const uint32_t r = scan[32 + wave] + x - v;
  *total = scan[63];
  __syncthreads();
  return r;
}

// Best K of keys[0..N) -> sm.out[0..K) sorted by (key desc, id asc); out[K..512) = 0.
__device__ void select_sorted(const TkShared& sm, int N, int K, int32_t id_base) {
  const int tid = threadIdx.x, wave = tid >> 6;
  __shared__ uint32_t sh_digit, sh_need;
  uint32_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)K;
  if (K > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < TK_WAVES * 256; i += TK_THREADS) sm.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < N; i += TK_THREADS) {
        const uint32_t k = sm.keys[i];
        if (((k ^ prefix) & mask) == 0) atomicAdd(&sm.hist[wave * 256 + ((k >> shift) & 255u)], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t c = 0;
        for (int w = 0; w < TK_WAVES; ++w) c += sm.hist[w * 256 + tid];
        sm.suf[tid] = c;
      }
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        uint32_t v = 0;
        if (tid < 256 && tid + off < 256) v = sm.suf[tid + off];
        __syncthreads();
        if (tid < 256) sm.suf[tid] += v;
        __syncthreads();
      }
      if (tid < 256) {
        const uint32_t above = tid < 255 ? sm.suf[tid + 1] : 0u;
        if (sm.suf[tid] >= need && above < need) {
          sh_digit = (uint32_t)tid;
          sh_need = need - above;
        }
      }
      __syncthreads();
      prefix |= sh_digit << shift;
      mask |= 255u << shift;
      need = sh_need;
      __syncthreads();
    }
  }
  const uint32_t T = prefix;
  // take: keys > T all, keys == T the first `need` in list order
  const int seg = (N + TK_THREADS - 1) / TK_THREADS;
  const int i0 = min(N, tid * seg), i1 = min(N, i0 + seg);
  uint32_t ngt = 0, neq = 0;
  if (K > 0)
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = sm.keys[i];
      ngt += k > T;
      neq += k == T;
    }
  uint32_t tot;
  uint32_t gt_off = block_excl_scan(ngt, sm.scan, &tot);
  uint32_t eq_off = block_excl_scan(neq, sm.scan, &tot);
  const uint32_t eq_base = (uint32_t)K - need;
  if (K > 0)
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = sm.keys[i];
      if (k < T) continue;
      const int32_t id = sm.ids ? sm.ids[i] : id_base + i;
      const unsigned long long comp = ((unsigned long long)k << 32) | (uint32_t)(~(uint32_t)id);
      if (k > T) {
        sm.out[gt_off++] = comp;
      } else {
        if (eq_off < need) sm.out[eq_base + eq_off] = comp;
        ++eq_off;
      }
    }
  for (int i = K + tid; i < TK; i += TK_THREADS) sm.out[i] = 0ull;
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= TK; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (tid < TK / 2) {
        const int i = ((tid & ~(j - 1)) << 1) | (tid & (j - 1));
        const int l = i + j;
        const unsigned long long a = sm.out[i], b = sm.out[l];
        const bool desc = (i & k) == 0;
        if (desc ? (a < b) : (a > b)) {
          sm.out[i] = b;
          sm.out[l] = a;
        }
      }
      __syncthreads();
    }
  }
}

__device__ inline TkShared carve(unsigned char* base, int nmax, bool with_ids) {
  TkShared s;
  s.out = reinterpret_cast<unsigned long long*>(base);
  s.hist = reinterpret_cast<uint32_t*>(base + TK * 8);
  s.suf = s.hist + TK_WAVES * 256;
  s.scan = s.suf + 256;
  s.keys = s.scan + 64;
  s.ids = with_ids ? reinterpret_cast<int32_t*>(s.keys + nmax) : nullptr;
  return s;
}

__host__ __device__ inline size_t tk_smem_bytes(int nmax, bool with_ids) {
  return (size_t)TK * 8 + (size_t)(TK_WAVES * 256 + 256 + 64) * 4 + (size_t)nmax * 4 * (with_ids ? 2 : 1);
}

__device__ inline int64_t unit_ncand(const int32_t* row_seq, const int64_t* row_pos, int64_t B,
                                     int64_t R_cap, int64_t pos_limit, int64_t row) {
  const int32_t s = row_seq[row];
  const int64_t p = row_pos[row];
  if (s < 0 || s >= B || p < 0 || p >= pos_limit || (p >> 3) > R_cap) return 0;
  return p >> 3;
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

// MODE 0: whole candidate range in one pass, final output.
// MODE 1: one chunk of the range, best 512 to `partial`.
__global__ __launch_bounds__(TK_THREADS) void topk_scores_kernel(
    int mode, const float* __restrict__ scores, int64_t R_cap, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, int64_t B, int64_t pos_limit, int64_t chunk, int nchunks,
    unsigned long long* __restrict__ partial, int32_t* __restrict__ sel_ids,
    float* __restrict__ sel_scores) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t unit = blockIdx.x;
  const int c = blockIdx.y;
  const TkShared sm = carve(smem, (int)chunk, false);
  const int64_t ncand = unit_ncand(row_seq, row_pos, B, R_cap, pos_limit, unit >> 2);
  const int64_t j0 = (int64_t)c * chunk;
  int N = 0;
  if (j0 < ncand) N = (int)((ncand - j0 < chunk) ? ncand - j0 : chunk);
  const float* src = scores + unit * R_cap + j0;
  for (int i = threadIdx.x; i < N; i += TK_THREADS) sm.keys[i] = ord_key(src[i]);
  __syncthreads();
  const int K = N < TK ? N : TK;
  select_sorted(sm, N, K, (int32_t)j0);
  if (mode == 0) {
    write_final(sm, K, unit, sel_ids, sel_scores);
  } else {
    unsigned long long* dst = partial + (unit * nchunks + c) * TK;
    for (int i = threadIdx.x; i < TK; i += TK_THREADS) dst[i] = sm.out[i];
  }
}

// Merge of the chunk lists of one (row, group): final output.
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(
    int64_t R_cap, const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_pos,
    int64_t B, int64_t pos_limit, int nchunks, const unsigned long long* __restrict__ partial,
    int32_t* __restrict__ sel_ids, float* __restrict__ sel_scores) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t unit = blockIdx.x;
  const int N = nchunks * TK;
  const TkShared sm = carve(smem, N, true);
  const int64_t ncand = unit_ncand(row_seq, row_pos, B, R_cap, pos_limit, unit >> 2);
  const unsigned long long* src = partial + unit * (int64_t)nchunks * TK;
  for (int i = threadIdx.x; i < N; i += TK_THREADS) {
    const unsigned long long c = src[i];
    sm.keys[i] = (uint32_t)(c >> 32);
    sm.ids[i] = (int32_t)(~(uint32_t)c);
  }
  __syncthreads();
  const int K = ncand < TK ? (int)ncand : TK;
  select_sorted(sm, N, K, 0);
  write_final(sm, K, unit, sel_ids, sel_scores);
}

TopkPlan topk_plan(int32_t rows, int64_t R_cap) {
  const int64_t units = (int64_t)rows * 4;
  const int64_t nmin = (R_cap + TK_MAX_N - 1) / TK_MAX_N;
  int64_t want = units > 0 ? (256 + units - 1) / units : 1;
  const int64_t by_size = (R_cap + 2047) / 2048;
  if (want > by_size) want = by_size;
  int64_t n = want > nmin ? want : nmin;
  if (n < 1) n = 1;
  if (n > TK_MAX_CHUNKS) n = TK_MAX_CHUNKS;
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
  const size_t sm1 = tk_smem_bytes((int)p.chunk, false);
  hipError_t e = hipFuncSetAttribute((const void*)topk_scores_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm1);
  if (e != hipSuccess) return e;
  if (p.nchunks == 1) {
    hipLaunchKernelGGL(topk_scores_kernel, dim3(units, 1), dim3(TK_THREADS), sm1, stream, 0,
                       a.scores, a.R_cap, a.row_seq, a.row_pos, a.B, a.pos_limit, p.chunk, 1,
                       (unsigned long long*)nullptr, a.sel_ids, a.sel_scores);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_scores_kernel, dim3(units, (unsigned)p.nchunks), dim3(TK_THREADS), sm1,
                     stream, 1, a.scores, a.R_cap, a.row_seq, a.row_pos, a.B, a.pos_limit, p.chunk, p.nchunks,
                     a.partial, (int32_t*)nullptr, (float*)nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t sm2 = tk_smem_bytes(p.nchunks * TK, true);
  e = hipFuncSetAttribute((const void*)topk_merge_kernel,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm2);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(units), dim3(TK_THREADS), sm2, stream, a.R_cap,
                     a.row_seq, a.row_pos, a.B, a.pos_limit, p.nchunks, (const unsigned long long*)a.partial,
                     a.sel_ids, a.sel_scores);
  return hipGetLastError();
}

}  // namespace s5
