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
// wave order, split states merge in split order: with up to 8 splits by the
// unit's last split to finish (an arrival counter per unit in the workspace;
// the split states are written and read through device-coherent memory, so no
// cache write-back is needed between workgroups on different dies), with more
// by a merge kernel (attn_mh_merge_kernel). Results are therefore independent
// of scheduling.
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
#include <atomic>

#include "attn_tile.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "step5.h"

namespace s5 {

constexpr int AT_ENTRIES = 513;  // own region + 512 selections
constexpr int AT_PART = 130;     // m, l, o[128] per head in a split state
constexpr int AT_MERGE_MAX = 8;  // splits merged inside the attention launch

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One 32-token chunk of a wave's list: K/V registers and the token counts of
// its four entries (8, the own region's p%8+1, or 0 for an empty slot).
struct AtChunk {
  uint4 k[2][4];
  uint4 v[8];
  bool kok[2];  // this lane's key token 16*st + n is present
};

// the i-th of four wave-uniform values, for a lane-dependent i
template <typename T>
__device__ inline T pick4(int i, T a, T b, T c, T d) {
  return i < 2 ? (i == 0 ? a : b) : (i == 2 ? c : d);
}

// Issues the loads of chunk `i` of this wave; entry e4 of the chunk is
// described by lane 4i+e4 of (lj, lcnt). Lanes whose token is absent load the
// row's own token (always in range) and are masked later.
__device__ __attribute__((always_inline)) inline void at_fetch(AtChunk& c, int i, int64_t lj, int lcnt, const uint16_t* kb,
                                const uint16_t* vb, int64_t kv_st, int64_t pc, int n, int qd) {
  int64_t jr[4];
  int cnt[4];
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    const int src = 4 * i + e4;
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)lj, src);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(lj >> 32), src);
    jr[e4] = (int64_t)(((uint64_t)hi << 32) | lo);
    cnt[e4] = __builtin_amdgcn_readlane(lcnt, src);
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int e4 = 2 * st + (n >> 3), ti = n & 7;
    const int ce = pick4(e4, cnt[0], cnt[1], cnt[2], cnt[3]);
    const int64_t je = pick4(e4, jr[0], jr[1], jr[2], jr[3]);
    c.kok[st] = ti < ce;
    const int64_t tok = c.kok[st] ? 8 * je + ti : pc;
    const uint16_t* kp = kb + tok * kv_st + 32 * qd;
#pragma unroll
    for (int u = 0; u < 4; ++u) c.k[st][u] = ldg16(kp + 8 * u);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int e4 = k >> 1, ti = 4 * (k & 1) + qd;  // e4 is the same in every lane
    const int64_t tok = (ti < cnt[e4]) ? 8 * jr[e4] + ti : pc;
    c.v[k] = ldg16(vb + tok * kv_st + 8 * n);
  }
}

struct AtState {
  float m[4], l[4], o[4][8];
};

// QK^T, online softmax and PV for one chunk.
__device__ __attribute__((always_inline)) inline void at_consume(const AtChunk& c, AtState& s, const uint4 (&qa)[4],
                                  float scale_log2, float4 (*p_w)[32], int n, int qd) {
  f32x4 acc[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    acc[st] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[st] = mfma_bf16(qa[u], c.k[st][u], acc[st]);
  }
  // lanes 0..15: acc[st][r] = score of head r with token 16*st + n
  float sv[2][4];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[st][r] = c.kok[st] ? acc[st][r] * scale_log2 : -INFINITY;
  }
  float alpha[4], pv[2][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float cmax = wave_uniform(max16_lanes(fmaxf(sv[0][r], sv[1][r])));
    const float mnew = fmaxf(s.m[r], cmax);
    const float mu = (mnew == -INFINITY) ? 0.f : mnew;
    alpha[r] = __builtin_amdgcn_exp2f(s.m[r] - mu);
    pv[0][r] = __builtin_amdgcn_exp2f(sv[0][r] - mu);
    pv[1][r] = __builtin_amdgcn_exp2f(sv[1][r] - mu);
    const float psum = wave_uniform(sum16_lanes(pv[0][r] + pv[1][r]));
    s.l[r] = s.l[r] * alpha[r] + psum;
    s.m[r] = mnew;
  }
  if (qd == 0) {
    (*p_w)[n] = make_float4(pv[0][0], pv[0][1], pv[0][2], pv[0][3]);
    (*p_w)[16 + n] = make_float4(pv[1][0], pv[1][1], pv[1][2], pv[1][3]);
  }
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) s.o[r][i] *= alpha[r];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 pw = (*p_w)[4 * k + qd];
    float vf[8];
    unpack_bf16x8(c.v[k], vf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s.o[0][i] = fmaf(pw.x, vf[i], s.o[0][i]);
      s.o[1][i] = fmaf(pw.y, vf[i], s.o[1][i]);
      s.o[2][i] = fmaf(pw.z, vf[i], s.o[2][i]);
      s.o[3][i] = fmaf(pw.w, vf[i], s.o[3][i]);
    }
  }
  wave_lds_sync();
}

__global__ __launch_bounds__(256) void attn_kernel(
    const uint16_t* __restrict__ q, int64_t qs, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t B, int64_t kv_sb, int64_t kv_st, int64_t T_cap,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, int32_t rows, int32_t sweep_maxr, float scale_log2,
    int per_split, int nsplit, float* __restrict__ partial, unsigned* __restrict__ arrive,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ float4 p_lds[4][32];            // per wave: P of 32 tokens, 4 heads each
  __shared__ float o_lds[4][4][4][128];      // [wave][token slot][head][dim]
  __shared__ float ml_lds[4][2][4];          // [wave][m | l][head]

  const int64_t unit = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t row = unit >> 2;
  const int g = (int)(unit & 3);
  if (sweep_maxr > 0) {
    // rows of a tile the context sweep (attn_tile_kernel) takes are its work
    int32_t sq;
    if (tl_tile_taken(row / TL_ROWS * TL_ROWS, rows, row_seq, row_pos, B, T_cap, sweep_maxr, &sq))
      return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;

  const int32_t seq = row_seq[row];
  const int64_t p = row_pos[row];
  const bool valid = seq >= 0 && seq < B && p >= 0 && p < T_cap;
  const int64_t ncand = valid ? (p >> 3) : 0;
  const int nent = valid ? 1 + (int)(ncand < 512 ? ncand : 512) : 0;
  const int e0 = split * per_split;
  const int e1 = min(e0 + per_split, nent);

  // this wave's entries: wb + 16 i + e4 (i < niter, e4 < 4); lane 4(i%16) + e4
  // describes one of them, the table reloaded every 16 chunks
  const int wb = e0 + 4 * wave;
  const int niter = wb < e1 ? (e1 - wb + 15) >> 4 : 0;
  const int32_t* sl = sel + unit * 512;
  __shared__ uint32_t ids_lds[512];
  if (nsplit == 1) {
    // one workgroup per unit (many rows: prefill): visit the selected regions
    // in id order, so the units resident on a chip die sweep the context
    // together and share its cached K/V lines; ids sort as unsigned (-1 last)
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
  int64_t lj;
  int lcnt;
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
  const int64_t pc = valid ? p : 0;  // a token that is always in range

  AtState s;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s.m[r] = -INFINITY;
    s.l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.o[r][i] = 0.f;
  }
  float4 (*p_w)[32] = &p_lds[wave];

  // two chunks in flight: the loads of chunk i+1 are issued before chunk i is
  // consumed
  AtChunk ca, cb;
  if (niter > 0) at_fetch(ca, 0, lj, lcnt, kb, vb, kv_st, pc, n, qd);
  for (int i = 0; i < niter; i += 2) {
    if (i + 1 < niter) {
      if (((i + 1) & 15) == 0) load_table(i + 1);
      at_fetch(cb, (i + 1) & 15, lj, lcnt, kb, vb, kv_st, pc, n, qd);
    }
    at_consume(ca, s, qa, scale_log2, p_w, n, qd);
    if (i + 1 >= niter) break;
    if (i + 2 < niter) {
      if (((i + 2) & 15) == 0) load_table(i + 2);
      at_fetch(ca, (i + 2) & 15, lj, lcnt, kb, vb, kv_st, pc, n, qd);
    }
    at_consume(cb, s, qa, scale_log2, p_w, n, qd);
  }

  // ---- merge the four waves (fixed order)
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ml_lds[wave][0][r] = s.m[r];
      ml_lds[wave][1][r] = s.l[r];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float4* dst = reinterpret_cast<float4*>(&o_lds[wave][qd][r][8 * n]);
    dst[0] = make_float4(s.o[r][0], s.o[r][1], s.o[r][2], s.o[r][3]);
    dst[1] = make_float4(s.o[r][4], s.o[r][5], s.o[r][6], s.o[r][7]);
  }
  __syncthreads();
  const int r = threadIdx.x >> 6;
  const int d0 = 2 * (threadIdx.x & 63);
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][0][r]);
  float Mu = (M == -INFINITY) ? 0.f : M;
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
  if (nsplit > 1) {
    // This split's state, stored with device-scope (write-through) stores. With
    // few splits (AT_MERGE_MAX; `arrive` given) the unit's last split merges
    // them: every thread waits for its stores, then one arrival per split at
    // the unit's counter; the last split to arrive resets the counter (the
    // workspace is left as found) and merges every split's state, read with
    // device-scope loads all issued at once, in split order. With more splits
    // attn_mh_merge_kernel merges them afterwards.
    __shared__ int sh_last;
    float* dst = partial + ((unit * nsplit + split) * 4 + r) * AT_PART;
    if (d0 == 0) {
      __hip_atomic_store(dst, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(dst + 2 + d0, O0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dst + 3 + d0, O1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!arrive) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned old = __hip_atomic_fetch_add(&arrive[unit], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == (unsigned)nsplit - 1u;
      if (last) __hip_atomic_store(&arrive[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh_last = last;
    }
    __syncthreads();
    if (!sh_last) return;
    const float* st = partial + (unit * nsplit * 4 + r) * AT_PART;
    const int64_t sstride = 4 * AT_PART;  // between a head's states of consecutive splits
    float mv[AT_MERGE_MAX], lv[AT_MERGE_MAX], ov0[AT_MERGE_MAX], ov1[AT_MERGE_MAX];
#pragma unroll
    for (int sp = 0; sp < AT_MERGE_MAX; ++sp) {
      if (sp < nsplit) {
        const float* ss = st + sp * sstride;
        mv[sp] = __hip_atomic_load(ss, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lv[sp] = __hip_atomic_load(ss + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ov0[sp] = __hip_atomic_load(ss + 2 + d0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ov1[sp] = __hip_atomic_load(ss + 3 + d0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < AT_MERGE_MAX; ++sp)
      if (sp < nsplit) M = fmaxf(M, mv[sp]);
    Mu = (M == -INFINITY) ? 0.f : M;
    L = 0.f;
    O0 = 0.f;
    O1 = 0.f;
#pragma unroll
    for (int sp = 0; sp < AT_MERGE_MAX; ++sp) {
      if (sp < nsplit) {
        const float f = __builtin_amdgcn_exp2f(mv[sp] - Mu);
        L = L + f * lv[sp];
        O0 = O0 + f * ov0[sp];
        O1 = O1 + f * ov1[sp];
      }
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const uint32_t packed = bf16_bits(O0 * inv) | (bf16_bits(O1 * inv) << 16);
  *reinterpret_cast<uint32_t*>(out + (row * 16 + 4 * g + r) * 128 + d0) = packed;
  if (lse && d0 == 0) lse[row * 16 + 4 * g + r] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

// Decode units are few (rows x 4): each gets enough splits for about
// S5_ATTN_BLOCKS workgroups in all, each split a multiple of 16 entries (four
// per wave per chunk); prefill units are many and run unsplit.
#ifndef S5_ATTN_BLOCKS
#define S5_ATTN_BLOCKS 256
#endif
AttnPlan attn_plan(int32_t rows) {
  const int64_t units = (int64_t)rows * 4;
  // more than one split only for fewer than S5_ATTN_BLOCKS units (the
  // workspace's counter region depends on it)
  int64_t ns = units > 0 ? (S5_ATTN_BLOCKS + units - 1) / units : 1;
  int64_t per = (AT_ENTRIES + ns - 1) / ns;
  per = (per + 15) / 16 * 16;
  if (per < 16) per = 16;
  AttnPlan a;
  a.per_split = (int32_t)per;
  a.nsplit = (int32_t)((AT_ENTRIES + per - 1) / per);
  return a;
}

// Workspace of a split call: one arrival counter per unit in a region of
// fixed size at the start (units are split only while there are fewer than
// S5_ATTN_BLOCKS of them, so the counters of every split call lie in it and
// no call's split states ever overlap them), then the split states.
constexpr size_t AT_COUNTER_BYTES = ((size_t)S5_ATTN_BLOCKS * sizeof(unsigned) + 255) / 256 * 256;

size_t attn_workspace_bytes(int32_t rows) {
  const AttnPlan a = attn_plan(rows);
  if (a.nsplit <= 1) return 0;
  return AT_COUNTER_BYTES + (size_t)rows * 4 * a.nsplit * 4 * AT_PART * sizeof(float);
}

// Many rows (a prompt chunk) go to the context sweep, tile by tile, when the
// contexts are at most S5_ATTN_TILE_MAX_REGIONS regions long; attn_kernel
// takes the rest. A tile's sweep takes as long whatever the row count (1.05
// ms per 4,096 regions on one CU), the gather about 0.68 us per row (both at
// 32K-token contexts), so the sweep pays from a full GPU's worth of tiles
// (2,048 rows) and up to about 5,400 regions.
#ifndef S5_ATTN_TILE_MIN_ROWS
#define S5_ATTN_TILE_MIN_ROWS 2048
#endif
#ifndef S5_ATTN_TILE_MAX_REGIONS
#define S5_ATTN_TILE_MAX_REGIONS 5120
#endif

// Scratch of step5_sparse_attn_noalloc (callers that cannot allocate): the
// split states of one call. Every GPU the library runs on holds its own copy
// of the array until the process ends; host code never passes the array's
// name to a kernel (on the host it is a stand-in, not a device address), only
// the address hipGetSymbolAddress gives on each device, kept per device.
// The split states are written in full before the merge reads them, so
// nothing in it needs clearing; calls that overlap on one GPU race on it.
__device__ __align__(256) unsigned char scratch[kAttnStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

int attn_static_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return STEP5_E_HIP;
  if (dev >= kMaxDevices) return STEP5_E_UNSUPPORTED;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return STEP5_E_HIP;
    if (sd != dev) return STEP5_E_INVALID;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return STEP5_E_HIP;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  *ptr = p;
  return STEP5_OK;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  if (a.qpk != 4 || a.head_dim != 128) return launch_attn_mh(a, stream);
  const AttnPlan pl = attn_plan(a.rows);
  int32_t maxr = 0;
  if (pl.nsplit == 1 && a.rows >= S5_ATTN_TILE_MIN_ROWS && a.T_cap > 0) {
    const int64_t nr = (a.T_cap + 7) / 8;
    maxr = (int32_t)(nr < S5_ATTN_TILE_MAX_REGIONS ? nr : S5_ATTN_TILE_MAX_REGIONS);
    // the sweep addresses a sequence's swept tokens with 32-bit byte offsets
    if ((int64_t)maxr * 8 * a.kv_st * 2 + 4096 >= INT32_MAX) maxr = 0;
    if (maxr > 0) {
      const hipError_t e = launch_attn_tile(a, maxr, stream);
      if (e != hipSuccess) return e;
    }
  }
  const unsigned units = (unsigned)a.rows * 4u;
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  unsigned* arrive = nullptr;
  float* states = nullptr;
  if (pl.nsplit > 1) {
    if (pl.nsplit <= AT_MERGE_MAX) arrive = reinterpret_cast<unsigned*>(a.partial);
    states = reinterpret_cast<float*>(reinterpret_cast<char*>(a.partial) + AT_COUNTER_BYTES);
  }
  hipLaunchKernelGGL(attn_kernel, dim3(units, (unsigned)pl.nsplit), dim3(256), 0, stream,
                     (const uint16_t*)a.q, a.q_stride_row, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.B, a.kv_sb, a.kv_st, a.T_cap, a.sel, a.row_seq,
                     a.row_pos, a.rows, maxr, scale_log2, pl.per_split, pl.nsplit, states,
                     arrive, (uint16_t*)a.out, a.lse);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit <= AT_MERGE_MAX) return e;
  // many splits (one or two rows): a merge kernel with one workgroup per
  // (unit, head) keeps every split's loads in flight; the states are laid out
  // as attn_mh.hip's, 4 heads x 128 dims
  return launch_attn_merge(states, pl.nsplit, a.rows, 4, 128, a.out, a.lse, stream);
}

}  // namespace s5
