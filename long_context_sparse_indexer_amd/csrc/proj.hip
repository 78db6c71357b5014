// The fused projection of a Step-5 full-attention layer: one product
// hidden @ W^T of the normed hidden state with a weight whose rows are
// [q | k | v | index_q | index_k | index_z | gate], its columns written
// straight into the seven outputs.
//
// vLLM, "vllm.models.step5.nvidia.model", class Step5FusedQKVIndexerLinear:
// both projections read the same normed hidden state, so one weight holds
// the attention's q/k/v rows followed by the indexer's q, k, z and the gate,
// and one GEMM replaces two; its split_indexer cuts the result by column.
// Here the cut is the GEMM's store: each 16-column tile of the output belongs
// to one part (every part is a multiple of 16 columns wide), so a tile's
// values go to that part's tensor at its own row stride, and no combined
// buffer exists.
//
// The product runs on the 16x16x32 bf16 MFMA as C^T = W hidden^T: weight
// rows (output columns) are the A operand, hidden rows the B operand, so a
// lane ends with 4 consecutive output columns of one row (an 8-byte store).
// fp32 accumulation, one rounding to bf16 at the end.
//  - proj_wide_kernel (many rows): 320 columns x 128 rows a workgroup (the
//    layer's 4,624 columns x 2,048 rows make 240 workgroups, one round on 256
//    CUs; 256-column tiles made 304, two rounds), 8 waves of 80 columns x 64
//    rows, the tiles of a chip die adjacent in column-tile order; k in steps
//    of 64 through LDS, double-buffered; tiles go from
//    memory straight into LDS (global_load_lds, 16 B a lane) with 16-byte
//    pieces XOR-swizzled by row so the fragment reads hit distinct banks.
//  - proj_narrow_kernel (a few rows, decode): the weight's 38 MB dominate, so
//    a workgroup takes 16 columns (289 workgroups at the layer's 4,624) and
//    its 4 waves split k, each streaming its quarter of the 16 weight rows
//    (hidden sizes 2,048 and 4,096: into LDS with global_load_lds, every
//    load instruction 4 rows x 256 contiguous bytes, two 128-k groups in
//    flight, fully unrolled; other sizes: registers, a loop); the four
//    partial tiles are summed in wave order (deterministic) through LDS.
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

namespace {

__device__ inline f32x4 pj_mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline void pj_load_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ inline void pj_wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// the part holding output column c (a multiple of 16) and c's column in it
__device__ inline int pj_part(const ProjOuts& o, int c) {
  int p = 0;
#pragma unroll
  for (int i = 1; i < PROJ_PARTS; ++i) p += c >= o.start[i] ? 1 : 0;
  return p;
}

// 4 fp32 -> 4 bf16 (nearest even) in 8 bytes
__device__ inline uint2 pj_pack4(f32x4 v) {
  return make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                    bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
}

constexpr int WD_BC = 320, WD_BR = 128, WD_BK = 64;  // wide tile
constexpr int WD_CB = WD_BC / 64;                  // 16-column blocks per wave (4 waves across)
constexpr int WD_PIECES = WD_BK / 8;                // 16-byte pieces per tile row

}  // namespace

// one stage of the wide kernel's LDS: [W tile 320 x 64 | hidden tile 128 x 64]
struct WdStage {
  uint4 v[(WD_BC + WD_BR) * WD_PIECES];
};

__global__ __launch_bounds__(512) void proj_wide_kernel(const uint16_t* __restrict__ h, int64_t hs,
                                                        int32_t rows, int32_t K,
                                                        const uint16_t* __restrict__ w, int32_t N,
                                                        ProjOuts o) {
  // two stages in separate arrays, so that reading one is seen not to
  // alias the loads landing in the other
  __shared__ WdStage st0, st1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, qd = lane >> 4;
  int bx, by;
  {
    // tiles of one 8-way round-robin slot (workgroup id mod 8, the chip die
    // the workgroup lands on) are consecutive in column-tile-major order, so
    // a die's workgroups share weight tiles through its L2
    const int ncol = (N + WD_BC - 1) / WD_BC, nrow = (rows + WD_BR - 1) / WD_BR, nt = ncol * nrow;
    const int L = blockIdx.x, per = (nt + 7) >> 3, r = nt & 7, x = L & 7, s = L >> 3;
    const int T = (r == 0 || x < r) ? x * per + s : r * per + (x - r) * (per - 1) + s;
    bx = T / nrow;
    by = T - bx * nrow;
  }
  const int c0 = bx * WD_BC, r0 = by * WD_BR;
  const int wc = wave & 3, wr = wave >> 2;  // this wave: columns 80 wc.., rows 64 wr..

  // staging: a wave's load fills 1 KB = 8 tile rows; lane -> (row l/8, slot l%8)
  // holding the row's piece slot ^ (row & 7). W tile: 40 such loads, hidden: 16.
  const int lrow = lane >> 3, lslot = lane & 7;
  const uint16_t* wsrc[WD_CB];
  const uint16_t* hsrc[2];
#pragma unroll
  for (int i = 0; i < WD_CB; ++i) {
    const int tr = 8 * WD_CB * wave + 8 * i + lrow;
    wsrc[i] = w + (int64_t)min(c0 + tr, N - 1) * K + 8 * (lslot ^ (tr & 7));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tr = 16 * wave + 8 * i + lrow;
    hsrc[i] = h + (int64_t)min(r0 + tr, rows - 1) * hs + 8 * (lslot ^ (tr & 7));
  }
  auto stage = [&](int kt, WdStage& sd) {
    const int k0 = kt * WD_BK;
#pragma unroll
    for (int i = 0; i < WD_CB; ++i)
      pj_load_lds16(wsrc[i] + k0, &sd.v[(8 * WD_CB * wave + 8 * i) * WD_PIECES]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      pj_load_lds16(hsrc[i] + k0, &sd.v[(WD_BC + 16 * wave + 8 * i) * WD_PIECES]);
  };

  f32x4 acc[WD_CB][4];
#pragma unroll
  for (int a = 0; a < WD_CB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const WdStage& sd) {
    const uint4* wl = &sd.v[0];
    const uint4* hl = &sd.v[WD_BC * WD_PIECES];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 af[WD_CB], bfr[4];
#pragma unroll
      for (int a = 0; a < WD_CB; ++a) {
        const int tr = 16 * WD_CB * wc + 16 * a + n;
        af[a] = wl[tr * WD_PIECES + ((4 * ks + qd) ^ (tr & 7))];
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int tr = 64 * wr + 16 * b + n;
        bfr[b] = hl[tr * WD_PIECES + ((4 * ks + qd) ^ (tr & 7))];
      }
#pragma unroll
      for (int a = 0; a < WD_CB; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = pj_mfma(af[a], bfr[b], acc[a][b]);
    }
  };

  // stage kt+1 loads while kt is consumed; one barrier per stage
  const int nk = K / WD_BK;
  stage(0, st0);
#pragma unroll 1
  for (int kt = 0; kt < nk; kt += 2) {
    pj_wait_loads();
    __syncthreads();
    if (kt + 1 < nk) stage(kt + 1, st1);
    compute(st0);
    if (kt + 1 >= nk) break;
    pj_wait_loads();
    __syncthreads();
    if (kt + 2 < nk) stage(kt + 2, st0);
    compute(st1);
  }

  // lane (n, qd) of tile (a, b): row 64 wr + 16 b + n, columns 80 wc + 16 a + 4 qd ..
#pragma unroll
  for (int a = 0; a < WD_CB; ++a) {
    const int ct = c0 + 16 * WD_CB * wc + 16 * a;  // the 16-column tile
    if (ct >= N) continue;
    const int p = pj_part(o, ct);
    const int cc = ct - o.start[p] + 4 * qd;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = r0 + 64 * wr + 16 * b + n;
      if (row < rows)
        *reinterpret_cast<uint2*>(o.ptr[p] + (int64_t)row * o.stride[p] + cc) = pj_pack4(acc[a][b]);
    }
  }
}

// one wave's group of 128 k in LDS: 16 weight rows then 16 hidden rows,
// 256 B each, 16-byte pieces XOR-swizzled by row
struct NrSlot {
  uint4 v[4][32 * 16];
};

// K = 512 GPW: each wave sums GPW groups of 128 k, its loads going straight
// into LDS (global_load_lds: one instruction reads 4 rows x 256 contiguous
// bytes), two groups in flight, fully unrolled.
template <int GPW>
__global__ __launch_bounds__(256) void proj_narrow_kernel(const uint16_t* __restrict__ h, int64_t hs,
                                                          int32_t rows, int32_t K,
                                                          const uint16_t* __restrict__ w, int32_t N,
                                                          ProjOuts o) {
  // the two slots in separate arrays, so that reading one is seen not to
  // alias the loads landing in the other
  __shared__ NrSlot sa, sb;
  __shared__ f32x4 red[3][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int c0 = blockIdx.x * 16, r0 = blockIdx.y * 16;
  const int kb = wave * (K / 4);
  // load j of a group: rows 4j + lane/16, lane -> slot lane%16 holding the
  // row's piece slot ^ row
  const int lr = lane >> 4, ls = lane & 15;
  const uint16_t* wsrc[4];
  const uint16_t* hsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * j + lr;
    wsrc[j] = w + (int64_t)(c0 + row) * K + kb + 8 * (ls ^ row);
    hsrc[j] = h + (int64_t)min(r0 + row, rows - 1) * hs + kb + 8 * (ls ^ row);
  }
  auto stage = [&](int g, NrSlot& sl) {
#pragma unroll
    for (int j = 0; j < 4; ++j) pj_load_lds16(wsrc[j] + 128 * g, &sl.v[wave][4 * j * 16]);
#pragma unroll
    for (int j = 0; j < 4; ++j) pj_load_lds16(hsrc[j] + 128 * g, &sl.v[wave][(16 + 4 * j) * 16]);
  };
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const NrSlot& sl) {
    const uint4* v = sl.v[wave];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int slot = (4 * st + qd) ^ n;
      acc = pj_mfma(v[n * 16 + slot], v[(16 + n) * 16 + slot], acc);
    }
  };
  stage(0, sa);
#pragma unroll
  for (int g = 0; g < GPW; ++g) {
    if (g + 1 < GPW) {
      if (g & 1) stage(g + 1, sa);
      else stage(g + 1, sb);
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // this group's 8 loads have landed
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if (g & 1) consume(sb);
    else consume(sa);
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    acc = ((acc + red[0][lane]) + red[1][lane]) + red[2][lane];
    const int p = pj_part(o, c0);
    const int row = r0 + n;
    if (row < rows)
      *reinterpret_cast<uint2*>(o.ptr[p] + (int64_t)row * o.stride[p] + (c0 - o.start[p]) + 4 * qd) =
          pj_pack4(acc);
  }
}

// any K (a multiple of 128): registers, a loop; pieces past a wave's range
// read as zero (a partial last group)
__global__ __launch_bounds__(256) void proj_narrow_any_kernel(const uint16_t* __restrict__ h, int64_t hs,
                                                              int32_t rows, int32_t K,
                                                              const uint16_t* __restrict__ w, int32_t N,
                                                              ProjOuts o) {
  __shared__ f32x4 red[3][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int c0 = blockIdx.x * 16, r0 = blockIdx.y * 16;
  const int kq = K / 4, kb = wave * kq, ng = (kq + 127) / 128;
  const uint16_t* wp = w + (int64_t)(c0 + n) * K + kb + 32 * qd;
  const uint16_t* hp = h + (int64_t)min(r0 + n, rows - 1) * hs + kb + 32 * qd;
  auto load = [&](int gi, uint4 (&wx)[4], uint4 (&hx)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = 128 * gi + 8 * s;
      const bool ok = k + 32 * qd < kq;
      wx[s] = ok ? ldg16(wp + k) : make_uint4(0u, 0u, 0u, 0u);
      hx[s] = ok ? ldg16(hp + k) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  uint4 wa[4], ha[4], wb[4], hb[4];
  load(0, wa, ha);
  load(1, wb, hb);
#pragma unroll 1
  for (int gi = 0; gi < ng; gi += 2) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = pj_mfma(wa[s], ha[s], acc);
    load(gi + 2, wa, ha);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = pj_mfma(wb[s], hb[s], acc);  // zero past the range
    load(gi + 3, wb, hb);
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    acc = ((acc + red[0][lane]) + red[1][lane]) + red[2][lane];
    const int p = pj_part(o, c0);
    const int row = r0 + n;
    if (row < rows)
      *reinterpret_cast<uint2*>(o.ptr[p] + (int64_t)row * o.stride[p] + (c0 - o.start[p]) + 4 * qd) =
          pj_pack4(acc);
  }
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int N = a.outs.start[PROJ_PARTS];
  if (a.rows >= S5_PROJ_WIDE_MIN_ROWS) {
    const dim3 grid((unsigned)(((N + WD_BC - 1) / WD_BC) * ((a.rows + WD_BR - 1) / WD_BR)));
    hipLaunchKernelGGL(proj_wide_kernel, grid, dim3(512), 0, stream, (const uint16_t*)a.hidden,
                       a.hidden_stride, a.rows, a.K, (const uint16_t*)a.weight, N, a.outs);
  } else {
    const dim3 grid((unsigned)(N / 16), (unsigned)((a.rows + 15) / 16));
    auto fn = a.K == 4096 ? proj_narrow_kernel<8> : a.K == 2048 ? proj_narrow_kernel<4>
                                                                 : proj_narrow_any_kernel;
    hipLaunchKernelGGL(fn, grid, dim3(256), 0, stream, (const uint16_t*)a.hidden, a.hidden_stride,
                       a.rows, a.K, (const uint16_t*)a.weight, N, a.outs);
  }
  return hipGetLastError();
}

}  // namespace s5
