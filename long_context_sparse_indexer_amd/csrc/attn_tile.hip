// Sparse attention for many rows of one sequence (a prompt chunk), 4 query
// heads per KV head of 128 dims: one sweep over the context per tile of 32
// rows and KV head, each row masked to its own selection.
//
// TensorFold #903 ("Step-5-Preview on one 256 GB Mac"): the indexer commit
// note attends over a row's selected regions and its own region up to the
// row's position; the commit note on chunked prompts runs the query heads
// through the MFMA against 32 keys at a time. Gathering each (row, KV head)'s
// 513 regions on its own reads 513 x 8 x 512 bytes of K and V per row from
// the cache hierarchy, although 32 consecutive rows of a prompt together
// select nearly every region of the context. Here a workgroup takes a tile
// of 32 rows and one KV head and reads the context once, in 32-token chunks:
// a chunk no row of the tile needs is skipped; inside a chunk, a row's scores
// for tokens outside its selected regions and its own region (up to its
// position) are -inf before its softmax. The result is the same attention as
// the per-row gather, up to summation order, wherever the K and V the tile's
// rows attend are finite: the rows of a tile share the staged chunk, so a
// NaN or inf in a token that one row attends also reaches the tile's other
// rows (through their -inf scores and zero probabilities), where the gather
// keeps rows apart. Tokens no row of the tile attends are staged as zero.
//
// Work per chunk, per wave (rows 4w .. 4w+3 of the tile; MFMA row n = row
// 4w + n/4, query head n%4):
//  - S^T = K Q^T on the 16x16x32 bf16 MFMA, K as the A operand from LDS and
//    the wave's queries as the B operand in registers; lane (n, qd) gets the
//    scores of MFMA row n for tokens 16 st + 4 qd + r;
//  - online softmax per MFMA row in the log2 domain. The running max is only
//    raised when a lane's probabilities for the chunk sum past 2^8 (so no
//    probability exceeds 2^8 otherwise; the result is the same up to
//    rounding), which makes the cross-lane max and the rescale of the
//    accumulators rare; the denominator is kept per lane and summed over the
//    row's 4 lanes at the end;
//  - O^T += V^T P^T, V^T as the A operand from LDS, P as the B operand
//    straight from the softmax registers (no LDS round trip): P is split into
//    its bf16 value and the bf16 of the remainder, two MFMAs, so P carries
//    about 16 bits.
// The sweep is pipelined over four LDS buffers with one barrier per chunk:
// step i stages chunk i+3 and, independently of each other, runs the output
// MFMAs of chunk i, the softmax of chunk i+1 and the score MFMAs of chunk i+2
// (the two waves sharing a SIMD take them in opposite orders). Staging uses
// buffer loads relative to a per-chunk base whose records end after the
// tile's last position (slots past it read as zero), and the K and V of
// tokens no row attends in the pass are stored as zero (so what such slots
// hold, inf or NaN included, never reaches a score or an output); K rows go
// to LDS as they are, in
// 16-byte pieces XOR-swizzled by token, V is written transposed (V^T[dim]
// [token]) with the 32 tokens of a dim in the order the P operand uses them.
// The chunk list is held in lane registers (64 ids a register), so a step
// reads no list entry from LDS. The rows' own regions, which need a causal
// cut inside the region, are attended after the sweep, one chunk each.
//
// The sweep takes only tiles whose valid rows share a sequence and whose own
// regions lie below a bound (tl_tile_taken); attn_kernel skips exactly those
// tiles' rows, so every row is computed once.
#include <type_traits>

#include "attn_tile.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace s5 {

namespace {

constexpr int TL_THREADS = 512;
constexpr int TL_D = 128;
constexpr float TL_M0 = -1e30f;   // running max before the first score (finite)
constexpr float TL_PMAX = 256.0f;  // raise the running max once a lane's chunk sum passes this

__device__ inline f32x4 tl_mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two floats -> two bf16 (nearest even) in one word, the first in the low half
__device__ inline uint32_t tl_pk(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}

// V^T row d: 4 pieces of 16 bytes (8 tokens each), piece slot XOR-swizzled
__device__ inline int tl_vsw(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
struct TlRegs {
  u32x4 k;
  u32x2 va, vb;
};


}  // namespace

size_t attn_tile_smem_bytes(int32_t maxr) { return tl_lds(maxr).total; }

__global__ __launch_bounds__(TL_THREADS) void attn_tile_kernel(
    const uint16_t* __restrict__ q, int64_t qs, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t B, int64_t kv_sb, int64_t kv_st, int64_t T_cap,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ row_seq,
    const int64_t* __restrict__ row_pos, int32_t rows, int32_t ntiles, int32_t maxr,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ __align__(16) unsigned char smem[];
  // workgroups go to the 8 chip dies in turn: dies 2g and 2g+1 take KV head
  // g, so a die's workgroups sweep the same K/V and share its L2
  const int xcd = blockIdx.x & 7;
  const int g = xcd >> 1;
  const int tile = 2 * (int)(blockIdx.x >> 3) + (xcd & 1);
  if (tile >= ntiles) return;
  const int64_t r0 = (int64_t)tile * TL_ROWS;
  int32_t seq;
  if (!tl_tile_taken(r0, rows, row_seq, row_pos, B, T_cap, maxr, &seq)) return;
  seq = __builtin_amdgcn_readfirstlane(seq);

  const TlLds L = tl_lds(maxr);
  uint4* kbuf = reinterpret_cast<uint4*>(smem);  // [4][512]
  uint4* vbuf = kbuf + 4 * 512;                  // [4][512]
  uint32_t* rmask = reinterpret_cast<uint32_t*>(smem + L.rmask);
  uint32_t* umask = reinterpret_cast<uint32_t*>(smem + L.umask);
  uint16_t* clist = reinterpret_cast<uint16_t*>(smem + L.clist);
  int64_t* rp = reinterpret_cast<int64_t*>(smem + L.rp);
  uint32_t* misc = reinterpret_cast<uint32_t*>(smem + L.misc);
  const int mw = (int)L.mw;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, qd = lane >> 4;

  // ---- the tile's rows and masks
  if (tid < TL_ROWS) {
    const int64_t r = r0 + tid;
    int64_t pv = -1;
    if (r < rows) {
      const int32_t s = row_seq[r];
      const int64_t p = row_pos[r];
      if (s >= 0 && s < B && p >= 0 && p < T_cap) pv = p;
    }
    rp[tid] = pv;
  }
  if (tid < 16 + 2 * TL_ROWS) misc[tid] = 0u;  // counters, own chunks, own token masks
  for (int w = tid; w < TL_ROWS * mw + (int)L.tw; w += TL_THREADS) rmask[w] = 0u;  // and umask
  __syncthreads();
  {
    // the rows' region bits: thread tid takes entry tid of every row's
    // selection (all 32 loads issued first), set by LDS atomics
    static_assert(TL_THREADS == 512, "one selection entry per thread and row");
    int32_t jr[TL_ROWS];
#pragma unroll
    for (int k = 0; k < TL_ROWS; ++k)
      jr[k] = r0 + k < rows ? sel[((r0 + k) * 4 + g) * 512 + tid] : -1;
#pragma unroll
    for (int k = 0; k < TL_ROWS; ++k) {
      const int64_t p = rp[k];
      const int32_t j = jr[k];
      if (p >= 0 && j >= 0 && j < (p >> 3)) atomicOr(&rmask[k * mw + (j >> 5)], 1u << (j & 31));
    }
  }
  if (tid < TL_ROWS && rp[tid] >= 0) {
    const int64_t p = rp[tid];
    atomicMax(&misc[0], (uint32_t)(p >> 3) + 1u);
    atomicMax(&misc[2], (uint32_t)p + 1u);
  }
  __syncthreads();
  // the tile's token mask per chunk: the union of the rows' region bits
  // (region word w holds chunks 8w .. 8w+7), each region's bit spread to its
  // 8 tokens (bit r of a nibble to byte r)
  for (int w = tid; w < mw; w += TL_THREADS) {
    uint32_t o = 0u;
    for (int k = 0; k < TL_ROWS; ++k) o |= rmask[k * mw + w];
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      const int c = 8 * w + c4;
      if (c < (int)L.tw) umask[c] = ((((o >> (4 * c4)) & 15u) * 0x00204081u) & 0x01010101u) * 0xffu;
    }
  }
  // the distinct chunks holding the rows' own regions (attended after the
  // sweep): row i's chunk unless an earlier row has it
  if (wave == 0) {
    const int64_t pi = lane < TL_ROWS ? rp[lane] : -1;
    bool first = pi >= 0;
    for (int j = 0; j < TL_ROWS; ++j) {
      const int64_t pj = rp[j];
      first = first && !(j < lane && pj >= 0 && (pj >> 5) == (pi >> 5));
    }
    const unsigned long long bal = __ballot(first);
    if (first) misc[16 + __popcll(bal & ((1ull << lane) - 1ull))] = (uint32_t)(pi >> 5);
    if (lane == 0) misc[3] = (uint32_t)__popcll(bal);
    // each row's tokens 8 (p/8) .. p into its chunk's token mask
    if (pi >= 0) {
      int j0 = lane;
      for (int j = TL_ROWS - 1; j >= 0; --j) {
        const int64_t pj = rp[j];
        if (j <= lane && pj >= 0 && (pj >> 5) == (pi >> 5)) j0 = j;
      }
      const int k = __popcll(bal & ((1ull << j0) - 1ull));
      const int jo = (int)(pi >> 3);
      atomicOr(&misc[16 + TL_ROWS + k], ((2u << (pi & 7)) - 1u) << (8 * (jo & 3)));
    }
  }
  __syncthreads();
  // the chunks holding some row's selected regions, in order
  const int nch_all = (int)((misc[0] + 3u) >> 2);
  for (int base = 0; base < nch_all; base += TL_THREADS) {
    const int c = base + tid;
    const bool need = c < nch_all && umask[c] != 0u;
    const unsigned long long bal = __ballot(need);
    if (lane == 0) misc[4 + wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t off = misc[1];
    for (int w = 0; w < wave; ++w) off += misc[4 + w];
    if (need) clist[off + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)c;
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < TL_THREADS / 64; ++w) tot += misc[4 + w];
      misc[1] += tot;
    }
    __syncthreads();
  }
  __syncthreads();
  const int nch = (int)misc[1];
  const int nown = (int)misc[3];

  // ---- this lane's MFMA row
  const int rl = 4 * wave + (n >> 2);
  const int h = n & 3;
  const int64_t prow = rp[rl];
  uint4 qb[4];
  {
    const uint16_t* qp = q + (r0 + rl) * qs + (4 * g + h) * TL_D + 8 * qd;
#pragma unroll
    for (int u = 0; u < 4; ++u) qb[u] = prow >= 0 ? ldg16(qp + 32 * u) : make_uint4(0, 0, 0, 0);
  }
  float ms = TL_M0, l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // ---- staging through buffer loads: a chunk's K and V rows relative to a
  // per-chunk base, with the records ending after the tile's last position,
  // so that slots past it read as zero. Thread: K piece kp of token kt; V
  // dims 8 vs + 4 vh .. +3 of tokens 2 vi and 2 vi + 1.
  const int kt = tid >> 4, kp = tid & 15;
  const int vi = tid & 15, vh = (tid >> 4) & 1, vs = tid >> 5;
  const int64_t tok_bytes = 2 * kv_st;
  const unsigned char* kbase =
      reinterpret_cast<const unsigned char*>(kc + (int64_t)seq * kv_sb + (int64_t)g * TL_D);
  const unsigned char* vbase =
      reinterpret_cast<const unsigned char*>(vc + (int64_t)seq * kv_sb + (int64_t)g * TL_D);
  const uint32_t pend = (uint32_t)__builtin_amdgcn_readfirstlane((int)misc[2]);  // last position + 1
  const int64_t rec_end = (int64_t)(pend > 0u ? pend - 1u : 0u) * tok_bytes + 2 * TL_D;
  const uint32_t ko = (uint32_t)(kt * tok_bytes + 16 * kp);
  const uint32_t vo0 = (uint32_t)(2 * vi * tok_bytes + 2 * (8 * vs + 4 * vh));
  const uint32_t vo1 = vo0 + (uint32_t)tok_bytes;
  auto load_chunk = [&](int c) {
    const int64_t off = (int64_t)c * 32 * tok_bytes;
    const int64_t left = rec_end - off;
    const int nrec = left > 0 ? (int)left : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + off), (short)0, nrec, RAW_RSRC3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + off), (short)0, nrec, RAW_RSRC3);
    TlRegs R;
    R.k = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)ko, 0, 0);
    R.va = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)vo0, 0, 0);
    R.vb = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)vo1, 0, 0);
    return R;
  };
  // tokens 2vi, 2vi+1 sit at positions k, k+1 of the operand order
  // k = 8 ((t >> 2) & 3) + 4 (t >> 4) + (t & 3): piece (t >> 2) & 3 of the
  // row, dword 2 (t >> 4) + ((t >> 1) & 1) in it. Store j of a thread writes
  // dim 8 vs + 4 vh + (j ^ vh), so that each store's four rows are two even
  // and two odd ones (the two halves of the banks).
  const int vpiece = (vi >> 1) & 3, vdw = 2 * (vi >> 3) + (vi & 1);
  uint32_t vwo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = 8 * vs + 4 * vh + (j ^ vh);
    vwo[j] = (uint32_t)(d * 64 + 16 * (vpiece ^ tl_vsw(d)) + 4 * vdw);
  }
  // dims e even / odd take the low / high halves of the two tokens' words
  const uint32_t sel_even = vh ? 0x07060302u : 0x05040100u;
  const uint32_t sel_odd = vh ? 0x05040100u : 0x07060302u;
  const int kwo = kt * 16 + (kp ^ (kt & 15));
  // um: the chunk's tokens some row attends in this pass; K and V of the
  // others are stored as zero, so whatever their slots hold never reaches
  // a score or an output
  auto write = [&](const TlRegs& R, uint32_t um, int bf) {
    uint4 k = __builtin_bit_cast(uint4, R.k);
    uint32_t a0 = R.va.x, a1 = R.va.y, b0 = R.vb.x, b1 = R.vb.y;
    if (um != 0xffffffffu) {  // uniform: most chunks of a prompt are attended throughout
      const bool okk = (um >> kt) & 1u;
      const bool oka = (um >> (2 * vi)) & 1u, okb = (um >> (2 * vi + 1)) & 1u;
      k = okk ? k : make_uint4(0u, 0u, 0u, 0u);
      a0 = oka ? a0 : 0u;
      a1 = oka ? a1 : 0u;
      b0 = okb ? b0 : 0u;
      b1 = okb ? b1 : 0u;
    }
    kbuf[bf * 512 + kwo] = k;
    unsigned char* vd = reinterpret_cast<unsigned char*>(vbuf + bf * 512);
    *reinterpret_cast<uint32_t*>(vd + vwo[0]) = __builtin_amdgcn_perm(b0, a0, sel_even);
    *reinterpret_cast<uint32_t*>(vd + vwo[1]) = __builtin_amdgcn_perm(b0, a0, sel_odd);
    *reinterpret_cast<uint32_t*>(vd + vwo[2]) = __builtin_amdgcn_perm(b1, a1, sel_even);
    *reinterpret_cast<uint32_t*>(vd + vwo[3]) = __builtin_amdgcn_perm(b1, a1, sel_odd);
  };
  const uint32_t* rmrow = rmask + rl * mw;

  // S^T of the chunk in buffer bf: lane (n, qd), acc[st][r] = score of MFMA
  // row n with token 16 st + 4 qd + r (region 2 st + qd/2 of the chunk, token
  // 4 (qd & 1) + r in it); the two 4-MFMA chains alternate
  auto scores = [&](int bf, f32x4 (&acc)[2]) {
    const uint4* kl = kbuf + bf * 512;
    uint4 kf[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 4; ++u) kf[st][u] = kl[(16 * st + n) * 16 + ((4 * u + qd) ^ n)];
    acc[0] = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[1] = acc[0];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int st = 0; st < 2; ++st) acc[st] = tl_mfma(kf[st][u], qb[u], acc[st]);
  };
  // t = scale*log2(e)*score - ms where the row attends the token, else -inf:
  // in the sweep, the row's selected regions (whole regions)
  auto mask_bits = [&](int c) { return (rmrow[c >> 3] >> (4 * (c & 7))) & 15u; };
  auto masked_sel = [&](uint32_t mb, const f32x4 (&acc)[2], float (&t)[2][4]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const float bias = ((mb >> (2 * st + (qd >> 1))) & 1u) ? -ms : -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[st][r] = fmaf(acc[st][r], scale_log2, bias);
    }
  };
  // after it, the row's own region up to its position
  auto masked_own = [&](int c, const f32x4 (&acc)[2], float (&t)[2][4]) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = 32 * (int64_t)c + 16 * st + 4 * qd + r;
        const bool ok = prow >= 0 && (tok >> 3) == (prow >> 3) && tok <= prow;
        t[st][r] = ok ? fmaf(acc[st][r], scale_log2, -ms) : -INFINITY;
      }
  };
  // probabilities, their lane sum, and the P^T operand (element
  // k = 8 qd + 4 st + r) as bf16 values and the bf16 of the remainders
  auto probs = [&](const float (&t)[2][4], uint4& phi, uint4& plo) {
    float p[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[st][r] = __builtin_amdgcn_exp2f(t[st][r]);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int st = i >> 1, r = 2 * (i & 1);
      hw[i] = tl_pk(p[st][r], p[st][r + 1]);
      lw[i] = tl_pk(p[st][r] - bf_lo(hw[i]), p[st][r + 1] - bf_hi(hw[i]));
    }
    phi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    plo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    return ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
  };
  // end of a softmax step (ps = probs(t, ...)): the running max is raised,
  // and the accumulators rescaled, only when some lane's chunk sum passes
  // 2^8 (so no probability does otherwise); the accumulators must hold every
  // earlier chunk when this runs
  auto settle = [&](float (&t)[2][4], const f32x4 (&acc)[2], float ps, uint4& phi, uint4& plo) {
    if (__ballot(!(ps <= TL_PMAX)) != 0ull) {
      float am = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = t[st][r] == -INFINITY ? -INFINITY : acc[st][r] * scale_log2;
          am = fmaxf(am, a);
        }
      am = fmaxf(am, __shfl_xor(am, 16));
      am = fmaxf(am, __shfl_xor(am, 32));
      const float mn = fmaxf(ms, am);
      const float alpha = __builtin_amdgcn_exp2f(ms - mn);
      l *= alpha;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[ct][r] *= alpha;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t[st][r] != -INFINITY) t[st][r] = fmaf(acc[st][r], scale_log2, -mn);
      ms = mn;
      ps = probs(t, phi, plo);
    }
    l += ps;
  };
  // O^T += V^T P^T for the chunk in buffer bf
  auto pv = [&](int bf, const uint4& phi, const uint4& plo) {
    const uint4* vl = vbuf + bf * 512;
    uint4 vf[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int d = 16 * ct + n;
      vf[ct] = vl[d * 4 + (qd ^ tl_vsw(d))];
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      o[ct] = tl_mfma(vf[ct], phi, o[ct]);
      o[ct] = tl_mfma(vf[ct], plo, o[ct]);
    }
  };

  // ---- the sweep. Chunk ci lives in LDS buffer ci % 4 (the loop is unrolled
  // by 4 so buffer offsets are constants). Step ci: one barrier; the staging
  // registers (chunk ci+3) go to buffer (ci+3) % 4 and chunk ci+4 is loaded;
  // then three independent pieces of work, their instructions interleaved:
  // the output MFMAs of chunk ci, the softmax of chunk ci+1 (scores from the
  // step before) and the score MFMAs of chunk ci+2.
  TlRegs R;
  uint32_t umR = 0;  // token mask of the chunk in R
  uint4 phi, plo;
  f32x4 acc1[2];
  // chunk ids and token masks from registers: lane i of clv0 (clu0) holds
  // the id (token mask) of list entry 64 clb + i, clv1 (clu1) those of the
  // next 64 (no LDS round trip, and no wait for one, per step)
  uint32_t clv0 = 0, clv1 = 0, clu0 = 0, clu1 = 0;
  int clb = 0;
  auto cl_fetch = [&](int blk) { const int i = 64 * blk + lane; return i < nch ? (uint32_t)clist[i] : 0u; };
  auto cu_fetch = [&](int blk) {
    const int i = 64 * blk + lane;
    return i < nch ? umask[clist[i]] : 0u;
  };
  auto cid = [&](int i) {
    const int a = __builtin_amdgcn_readlane((int)clv0, i & 63);
    const int b = __builtin_amdgcn_readlane((int)clv1, i & 63);
    return (i >> 6) == clb ? a : b;
  };
  auto cum = [&](int i) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)clu0, i & 63);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)clu1, i & 63);
    return (i >> 6) == clb ? a : b;
  };
  uint32_t mb1 = 0;  // this row's region bits in chunk ci+1 (read a step ahead)
  auto step = [&](auto b0c, int ci) {
    constexpr int B0 = decltype(b0c)::value, B2 = (B0 + 2) % 4, B3 = (B0 + 3) % 4;
    if (ci > 0) __syncthreads();
    if ((ci & 63) == 0 && ci > 0) {
      clv0 = clv1;
      clv1 = cl_fetch((ci >> 6) + 1);
      clu0 = clu1;
      clu1 = cu_fetch((ci >> 6) + 1);
      clb = ci >> 6;
    }
    const uint32_t mb2 = mask_bits(cid(min(ci + 2, nch - 1)));
    if (ci + 3 < nch) {
      write(R, umR, B3);
      R = load_chunk(cid(min(ci + 4, nch - 1)));
      umR = cum(min(ci + 4, nch - 1));
    }
    if (ci + 1 < nch) {
      // the two waves sharing a SIMD (w and w + 4) take the matrix work and
      // the softmax in opposite orders, so one feeds the MFMA unit while the
      // other runs vector instructions. In the matrix work the scores' 8
      // operand reads from LDS are issued together, then their 8 MFMAs,
      // then the output's 8 reads and 16 MFMAs (the scheduling groups below:
      // left alone, the compiler reuses a few registers and waits on each read)
      f32x4 acc2[2];
      float t[2][4];
      uint4 nhi, nlo;
      float ps;
      if (wave & 4) {
        masked_sel(mb1, acc1, t);
        ps = probs(t, nhi, nlo);
        __builtin_amdgcn_sched_barrier(0);
        scores(B2, acc2);  // chunk ci+2 (unused past the last chunk)
        pv(B0, phi, plo);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      } else {
        scores(B2, acc2);
        pv(B0, phi, plo);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        __builtin_amdgcn_sched_barrier(0);
        masked_sel(mb1, acc1, t);
        ps = probs(t, nhi, nlo);
      }
      settle(t, acc1, ps, nhi, nlo);
      phi = nhi;
      plo = nlo;
      acc1[0] = acc2[0];
      acc1[1] = acc2[1];
    } else {
      pv(B0, phi, plo);
    }
    mb1 = mb2;
  };
  if (nch > 0) {
    clv0 = cl_fetch(0);
    clv1 = cl_fetch(1);
    clu0 = cu_fetch(0);
    clu1 = cu_fetch(1);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int c = cid(min(i, nch - 1));
      write(load_chunk(c), umask[c], i);
    }
    R = load_chunk(cid(min(3, nch - 1)));
    umR = umask[cid(min(3, nch - 1))];
    __syncthreads();
    f32x4 acc[2];
    scores(0, acc);
    float t[2][4];
    masked_sel(mask_bits(cid(0)), acc, t);
    const float ps = probs(t, phi, plo);
    settle(t, acc, ps, phi, plo);
    scores(1, acc1);
    mb1 = mask_bits(cid(min(1, nch - 1)));
#pragma unroll 1
    for (int ci = 0; ci < nch; ci += 4) {
      step(std::integral_constant<int, 0>(), ci);
      if (ci + 1 >= nch) break;
      step(std::integral_constant<int, 1>(), ci + 1);
      if (ci + 2 >= nch) break;
      step(std::integral_constant<int, 2>(), ci + 2);
      if (ci + 3 >= nch) break;
      step(std::integral_constant<int, 3>(), ci + 3);
    }
  }
  // ---- the rows' own regions, chunk by chunk
#pragma unroll 1
  for (int k = 0; k < nown; ++k) {
    const int c = __builtin_amdgcn_readfirstlane((int)misc[16 + k]);
    const uint32_t um = (uint32_t)__builtin_amdgcn_readfirstlane((int)misc[16 + TL_ROWS + k]);
    __syncthreads();
    write(load_chunk(c), um, 0);
    __syncthreads();
    f32x4 acc[2];
    scores(0, acc);
    float t[2][4];
    masked_own(c, acc, t);
    uint4 ohi, olo;
    const float ps = probs(t, ohi, olo);
    settle(t, acc, ps, ohi, olo);
    pv(0, ohi, olo);
  }

  // ---- outputs: lane (n, qd) holds dims 16 ct + 4 qd + r of MFMA row n
  float L2 = l + __shfl_xor(l, 16);
  L2 = L2 + __shfl_xor(L2, 32);
  const int64_t row = r0 + rl;
  if (row < rows) {
    const float inv = L2 > 0.f ? 1.0f / L2 : 0.f;
    uint16_t* dst = out + (row * 16 + 4 * g + h) * TL_D + 4 * qd;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint2 w = make_uint2(bf16_bits(o[ct][0] * inv) | (bf16_bits(o[ct][1] * inv) << 16),
                                 bf16_bits(o[ct][2] * inv) | (bf16_bits(o[ct][3] * inv) << 16));
      *reinterpret_cast<uint2*>(dst + 16 * ct) = w;
    }
    if (lse && qd == 0)
      lse[row * 16 + 4 * g + h] = L2 > 0.f ? (ms + log2f(L2)) * 0.6931471805599453f : -INFINITY;
  }
}

hipError_t launch_attn_tile(const AttnArgs& a, int32_t maxr, hipStream_t stream) {
  const int32_t ntiles = (a.rows + TL_ROWS - 1) / TL_ROWS;
  const unsigned blocks = 8u * (unsigned)((ntiles + 1) / 2);
  const size_t sm = attn_tile_smem_bytes(maxr);
  hipError_t e = hipFuncSetAttribute((const void*)attn_tile_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  hipLaunchKernelGGL(attn_tile_kernel, dim3(blocks), dim3(TL_THREADS), sm, stream,
                     (const uint16_t*)a.q, a.q_stride_row, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.B, a.kv_sb, a.kv_st, a.T_cap, a.sel, a.row_seq,
                     a.row_pos, a.rows, ntiles, maxr, scale_log2, (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

}  // namespace s5
