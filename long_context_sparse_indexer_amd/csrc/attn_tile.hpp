// Shared by attn_tile.hip (the context sweep over 32-row tiles) and attn.hip
// (the per-unit gather): which tiles the sweep takes, and its LDS layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s5 {

constexpr int TL_ROWS = 32;  // rows per tile

// Byte offsets of the sweep kernel's LDS for `maxr` regions:
//   K and V^T buffers for 4 chunks (4 x 2 x 8 KB), per-row region bitmasks
//   [32][mw], the tile's token bitmask [tw] (one word per 32-token chunk),
//   the needed-chunk list [tw] (u16), row positions [32], counters [16], the
//   chunks of the rows' own regions [32] and their token masks [32].
struct TlLds {
  uint32_t mw, tw, rmask, umask, clist, rp, misc, total;
};
__host__ __device__ inline TlLds tl_lds(int32_t maxr) {
  TlLds L;
  L.mw = (uint32_t)(maxr + 31) / 32;
  L.tw = (uint32_t)(maxr + 3) / 4;
  uint32_t o = 4 * 2 * 512 * 16;
  L.rmask = o;
  o += TL_ROWS * L.mw * 4;
  L.umask = o;
  o += L.tw * 4;
  L.clist = o;
  o += (L.tw * 2 + 15) / 16 * 16;
  L.rp = o;
  o += TL_ROWS * 8;
  L.misc = o;
  o += (16 + 2 * TL_ROWS) * 4;
  L.total = o;
  return L;
}

// Whether the sweep takes the tile of rows r0 .. r0+31: its valid rows
// (sequence in 0..B-1, position in 0..T_cap-1) share one sequence and their
// own regions lie below `maxr`. A tile without valid rows is taken. Called by
// a whole wave; lanes 0..31 read the rows; the result is wave-uniform. `seq`
// receives the shared sequence (0 if none).
__device__ inline bool tl_tile_taken(int64_t r0, int32_t rows, const int32_t* row_seq,
                                     const int64_t* row_pos, int64_t B, int64_t T_cap,
                                     int32_t maxr, int32_t* seq) {
  const int lane = threadIdx.x & 63;
  const int64_t r = r0 + lane;
  bool valid = false;
  int32_t s = 0;
  int64_t p = 0;
  if (lane < TL_ROWS && r < rows) {
    s = row_seq[r];
    p = row_pos[r];
    valid = s >= 0 && s < B && p >= 0 && p < T_cap;
  }
  const unsigned long long vb = __ballot(valid);
  *seq = 0;
  if (vb == 0ull) return true;
  const int32_t s0 = __shfl(s, __builtin_ctzll(vb));
  *seq = s0;
  return __ballot(valid && (s != s0 || (p >> 3) >= maxr)) == 0ull;
}

}  // namespace s5
