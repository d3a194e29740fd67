// prefill.hip -- window / paired-half-segment attention forward for gfx950.
//
// One workgroup (4 waves) owns a block of 128 consecutive query rows of one
// (batch, head); each wave owns 32 of them.  Key/value tiles (64 rows for
// d = 64, 32 rows for d = 128) stream through LDS; the workgroup walks the
// tiles covering the union of its rows' key ranges:
//   window (pi-Attention section 2 item 1; LT2 section 2.1): [max(0,i-k), i]
//   ECP (PAR block, ECP section 2):       [max(0,(floor(i/s)-1)*s), i]
//   and the further masks (two-sided window, s-Split segments, ECP pair
//   without the causal mask), each a range [key_lo(i), key_hi(i)].
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// every lane then owns ONE query and 32 keys of the tile, so the softmax row
// max and sum are lane-local plus one exchange between the wave halves
// (v_permlane32_swap).  P^T stays in registers as the B operand of
// O^T = V^T P^T; the V^T fragment comes straight from the row-major V tile
// through ds_read_b64_tr_b16.
//
// Pipelining (bf16): K/V tiles are double-buffered in LDS and loaded straight
// from HBM into LDS; while the waves compute on tile t, the direct-to-LDS
// loads of tile t+1 are in flight, and one barrier per tile hands the buffers
// over.  Without staging registers the d = 64 kernel fits 4 waves per SIMD.
//
// The softmax is online in log2 units against a lazily moved reference:
// exact, since numerator and denominator use the same reference.  The fp32
// kernel moves it when a tile raises the row max by more than 8; the bf16
// kernel takes the max only on a wave's first tile and afterwards checks the
// tile's probability sums instead (see the tile loop).
// For pi-Attention the periodic skip keys are handled by a separate pass
// (skip.hip) whose partial softmax state (max, sum, accumulator) seeds the
// running state here: the union gets one softmax, as the page requires.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;
constexpr float kTau = 8.0f;
// Largest lane sum of one tile's probabilities accepted without taking the
// row max (bf16 kernel): every probability is then at most 2^8.
constexpr float kSumCap = 256.0f;

struct Params {
  const void *q, *k, *v;
  const float *alpha;
  void *o;
  const float *skip_ml;
  const void *skip_acc;
  float *lse;             // [B*Hq*N] natural-log normaliser per row, or nullptr
  int N, Hq, Hkv, mode, k_win, seg, nqb, total, skip_first;
  int heads_per_xcd;   // > 0: heavy-first block order per XCD (see block_of)
  int rank_group;      // heads walked together in rank order (divides heads_per_xcd)
  int ecp_J, ecp_C;    // ECP blocks per half-segment and half-segments (0: none)
  float scale_log2;
  FusedOpts opt;
};

// Gate and epilogue helpers shared by both prefill kernels.
__device__ __forceinline__ float sigmoidf_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
}

// log2(sigmoid(z)) without overflow for large |z|.
__device__ __forceinline__ float log2_sigmoid(float z) {
  return z >= 0.f ? -__log2f(1.0f + fast_exp2(-z * kLog2e)) : z * kLog2e - __log2f(1.0f + fast_exp2(z * kLog2e));
}


// Work order.  A query block's cost is its number of key tiles, which varies
// with the block: ECP blocks in half-segment 0 and early in a half-segment are
// light, causal window blocks near position 0 are light.  Blocks are handed
// out heaviest first, so the light ones fill the grid's tail (list scheduling
// by decreasing cost).  The grid is split into 8 contiguous ranges, one per
// XCD (xcd_remap); each XCD owns heads_per_xcd whole heads and walks them in
// groups of rank_group heads whose K/V fit in its L2, each group in cost rank
// order: all the group's heaviest blocks, then the next, and so on.
// Otherwise (heads not a multiple of 8, or block costs nearly equal) each
// head's blocks run last-to-first.
struct BlockId {
  int bh, qb;
};

__device__ __forceinline__ BlockId block_of(const Params &p, int bid) {
  const int logical = xcd_remap(bid, p.total);
  BlockId r;
  if (p.heads_per_xcd <= 0) {
    r.qb = p.nqb - 1 - logical % p.nqb;
    r.bh = logical / p.nqb;
    return r;
  }
  const int per = p.total / 8;
  const int x = logical / per, idx = logical - x * per;
  const int gsz = p.rank_group * p.nqb;                 // blocks of one head group
  const int grp = idx / gsz, rem = idx - grp * gsz;
  const int rank = rem / p.rank_group;
  r.bh = x * p.heads_per_xcd + grp * p.rank_group + (rem - rank * p.rank_group);
  if (p.ecp_J > 0) {
    // ECP with whole half-segments: cost depends on the block's position j in
    // its half-segment (heavier later) and on c > 0.
    const int J = p.ecp_J, C = p.ecp_C;
    int j, c;
    if (rank < J * (C - 1)) {
      j = J - 1 - rank / (C - 1);
      c = 1 + rank % (C - 1);
    } else {
      j = J - 1 - (rank - J * (C - 1));
      c = 0;
    }
    r.qb = c * J + j;
  } else {
    r.qb = p.nqb - 1 - rank;
  }
  return r;
}



// fp32 I/O (small problems, exact-arithmetic checks): the same walk over key
// tiles with v_mfma_f32_32x32x2f32, one LDS buffer (rows padded by 16 bytes)
// and plain 4-byte operand reads.
template <int D>
__global__ __launch_bounds__(256, 2) void prefill_f32_kernel(Params p) {
  constexpr int LD = D + 4;                 // floats per LDS row
  constexpr int CPR = D / 4;                // 16-byte chunks per row
  constexpr int PER_THREAD = BN * CPR / 256;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) float Ks[BN * LD];
  __shared__ __attribute__((aligned(16))) float Vs[BN * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const BlockId blk = block_of(p, blockIdx.x);
  const int qb = blk.qb, bh = blk.bh;
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int g = hq / (p.Hq / p.Hkv);
  const int N = p.N;
  const int i0 = qb * BM, q0 = i0 + wave * 32, qi = q0 + c;
  const bool qvalid = qi < N;

  const float *Qp = (const float *)p.q + (size_t)bh * N * D;
  const float *Kp = (const float *)p.k + (size_t)(b * p.Hkv + g) * N * D;
  const float *Vp = (const float *)p.v + (size_t)(b * p.Hkv + g) * N * D;

  const int lo_i = key_lo(qi, p.mode, p.k_win, p.seg);
  float bias = 0.f;  // log2 of the local prior
  if (p.mode == kModePi && p.alpha != nullptr && p.opt.gate_w == nullptr && qvalid)
    bias = __log2f(p.alpha[(size_t)bh * N + qi]);

  float qf[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qf[kk] = qvalid ? Qp[(size_t)qi * D + 2 * kk + h] : 0.f;
  float sl2 = p.scale_log2;
  if (p.opt.cosine) {   // scale * cos(q, k): keys arrive normalised, 1/|q_i| joins this lane's scale
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) ss = fmaf(qf[kk], qf[kk], ss);
    sl2 *= rsqrtf(half_swap_sum(ss));
  }
  if (p.opt.gate_w != nullptr && p.mode == kModePi) {   // alpha = sigmoid(<w_h, q_i> + b_h)
    const int hg = (p.opt.gate_bh0 + bh) % p.opt.gate_hq;
    const float *w = p.opt.gate_w + (size_t)hg * D;
    float z = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) z = fmaf(qf[kk], w[2 * kk + h], z);
    bias = log2_sigmoid(half_swap_sum(z) + p.opt.gate_b[hg]);
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;

  // Seed with the skip-key partial state (pi-Attention union, one softmax).
  if (p.skip_ml != nullptr && qvalid && qi >= p.skip_first) {
    const size_t row = (size_t)bh * N + qi;
    m_run = p.skip_ml[2 * row];
    if (h == 0) l_run = p.skip_ml[2 * row + 1];
    const float *ap = (const float *)p.skip_acc + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 x = *(const f32x4 *)(ap + 32 * db + 8 * j4 + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * j4 + e] = x[e];
      }
  }

  const int hi_i = key_hi(qi, N, p.mode, p.k_win, p.seg);
  const int hi_wg = key_hi(min(i0 + BM - 1, N - 1), N, p.mode, p.k_win, p.seg);
  const int t_begin = (key_lo(i0, p.mode, p.k_win, p.seg) / BN) * BN;
  const int ntiles = (hi_wg - t_begin) / BN + 1;
  const bool wave_live = q0 < N;
  const int w_hi = key_hi(min(q0 + 31, N - 1), N, p.mode, p.k_win, p.seg);
  const int w_lo = key_lo(min(q0, N - 1), p.mode, p.k_win, p.seg);

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t_begin + t * BN;
    __syncthreads();   // everyone is done with the previous tile
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int ci = tid + 256 * r;
      const int row = ci / CPR, col = (ci % CPR) * 4;
      const int key = min(j0 + row, N - 1);   // rows past N: masked / probability 0
      *(float4 *)&Ks[row * LD + col] = *(const float4 *)(Kp + (size_t)key * D + col);
      *(float4 *)&Vs[row * LD + col] = *(const float4 *)(Vp + (size_t)key * D + col);
    }
    __syncthreads();
    if (!(wave_live && j0 <= w_hi && j0 + BN - 1 >= w_lo)) continue;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const float *krow = Ks + (32 * kb + c) * LD;
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * kk + h], qf[kk], s[kb], 0, 0, 0);
    }
    // mask: key j visible to query i iff lo(i) <= j <= hi(i) (tile-local index
    // of register jj of block kb: 32kb + 8(jj/4) + 4h + jj%4)
    const int a0 = lo_i - j0 - 4 * h, span = hi_i - lo_i;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int off = 32 * kb + 8 * (jj >> 2) + (jj & 3);
        if ((unsigned)(off - a0) > (unsigned)span) s[kb][jj] = -INFINITY;
      }
    float mx = s[0][0];
#pragma unroll
    for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, s[0][jj]);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s[1][jj]);
    mx = half_swap_max(mx);
    const float m_new = mx * sl2 + bias;
    if (__any(m_new > m_run + kTau)) {
      const float mr = fmaxf(m_run, m_new);
      const float f = fast_exp2(m_run - mr);
      l_run *= f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= f;
      m_run = mr;
    }
    const float nb = bias - m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        s[kb][jj] = fast_exp2(fmaf(s[kb][jj], sl2, nb));
        l_run += s[kb][jj];
      }
    // O^T += V^T P^T: k index of the 32x32x2 product = lane half h <-> key
    // 32kb + 8(tt/4) + 4h + tt%4.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const float *vrow = Vs + (32 * kb + 8 * (tt >> 2) + 4 * h + (tt & 3)) * LD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db + c], s[kb][tt], acc[db], 0, 0, 0);
      }
  }

  const float l_tot = half_swap_sum(l_run);
  if (!qvalid) return;
  // Row normaliser (natural log): scores are carried in log2 units.
  if (p.lse != nullptr && h == 0) p.lse[(size_t)bh * N + qi] = (m_run + __log2f(l_tot)) * kLn2;
  const float inv = 1.0f / l_tot;
  float *op = (float *)p.o + ((size_t)bh * N + qi) * D;
  const float *gp = p.opt.out_gate != nullptr ? (const float *)p.opt.out_gate + ((size_t)bh * N + qi) * D : nullptr;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * j4 + e] * inv;
      if (gp != nullptr) {   // output gate o * sigmoid(g)
        const f32x4 gv = *(const f32x4 *)(gp + 32 * db + 8 * j4 + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] *= sigmoidf_fast(gv[e]);
      }
      *(f32x4 *)(op + 32 * db + 8 * j4 + 4 * h) = x;
    }
}


template <int D, int TBN>
__global__ __launch_bounds__(256, (D == 128 && TBN == 32) ? 3 : 2) void prefill_bf16_kernel(Params p) {
  constexpr int RB = D * 2;              // bytes per K/V row
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int NKB = TBN / 32;          // 32-key blocks per key tile
  constexpr int TILE = TBN * RB;         // bytes per K or V tile
  constexpr int PER_WAVE = TILE / 1024 / 4;  // DMA instructions per wave per tile
  constexpr int NQF = D / 16;            // k-steps of the 32x32x16 score product
  constexpr int NDB = D / 32;            // 32-dim blocks of O^T
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];   // K0 K1 V0 V1

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const BlockId blk = block_of(p, blockIdx.x);
  const int qb = blk.qb, bh = blk.bh;
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int g = hq / (p.Hq / p.Hkv);
  const int N = p.N;
  const int i0 = qb * BM, q0 = i0 + wave * 32, qi = q0 + c;
  const bool qvalid = qi < N;

  const bf16 *Qp = (const bf16 *)p.q + (size_t)bh * N * D;
  const bf16 *Kp = (const bf16 *)p.k + (size_t)(b * p.Hkv + g) * N * D;
  const bf16 *Vp = (const bf16 *)p.v + (size_t)(b * p.Hkv + g) * N * D;

  // ---- key-tile range ---------------------------------------------------
  const int hi_wg = key_hi(min(i0 + BM - 1, N - 1), N, p.mode, p.k_win, p.seg);
  const int t_begin = (key_lo(i0, p.mode, p.k_win, p.seg) / TBN) * TBN;
  const int ntiles = (hi_wg - t_begin) / TBN + 1;
  // Tile order.  Head-major windows start each block's walk at the tile
  // whose global index is 0 mod ntiles and wrap around, so that workgroups
  // running side by side (neighbouring blocks, ntiles equal) load the same
  // key tile at the same step and share it in L2 instead of each fetching it
  // at a different time.  Any order gives the same softmax (the masks are
  // per tile).
  int rot = 0;
  if (p.heads_per_xcd <= 0) {
    rot = (t_begin / TBN) % ntiles;
    rot = rot == 0 ? 0 : ntiles - rot;
  }
  auto tile_row = [&](int t) __attribute__((always_inline)) {
    int u = t + rot;
    if (u >= ntiles) u -= ntiles;
    return t_begin + u * TBN;
  };

  // ---- direct-to-LDS staging of one K and one V tile -----------------------
  // Lane L of DMA u carries 16 bytes of one tile row; the tile's first row j0
  // goes into the scalar address, so a tile lying wholly below N costs no
  // vector instructions (rows past N, in the last tile only, are clamped to
  // N - 1: masked or probability 0).
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  unsigned soff[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int pch = 64 * (PER_WAVE * wave + u) + lane;   // chunk position in LDS
    const int row = pch / CPR;
    soff[u] = (unsigned)(row * RB + (((pch % CPR) ^ tile_swz<D>(row)) << 4));
  }
  auto stage = [&](int j0, int buf) __attribute__((always_inline)) {
    const bf16 *kb = Kp + (size_t)j0 * D, *vb = Vp + (size_t)j0 * D;
    // (two loops, so that the clamp's vector arithmetic is not formed and
    // then discarded on every whole tile)
    if (j0 + TBN <= N) {
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const unsigned kdst = lds0 + buf * TILE + 1024 * (PER_WAVE * wave_s + u);
        dma16(kb, soff[u], kdst);
        dma16(vb, soff[u], kdst + 2 * TILE);
      }
    } else {
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const int row = (int)(soff[u] / RB);
        const unsigned off = soff[u] + (unsigned)((min(j0 + row, N - 1) - j0 - row) * RB);
        const unsigned kdst = lds0 + buf * TILE + 1024 * (PER_WAVE * wave_s + u);
        dma16(kb, off, kdst);
        dma16(vb, off, kdst + 2 * TILE);
      }
    }
  };
  // The first tile's loads go out before the query's, so the workgroup waits
  // once for both.
  stage(tile_row(0), 0);

  const int lo_i = key_lo(qi, p.mode, p.k_win, p.seg);
  float bias = 0.f;  // log2 of the local prior
  if (p.mode == kModePi && p.alpha != nullptr && p.opt.gate_w == nullptr && qvalid)
    bias = __log2f(p.alpha[(size_t)bh * N + qi]);

  bf16x8 qf[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk)
    qf[kk] = qvalid ? *(const bf16x8 *)(Qp + (size_t)qi * D + 16 * kk + 8 * h) : bf16x8{};
  float sl2 = p.scale_log2;
  if (p.opt.cosine) {   // scale * cos(q, k): keys arrive normalised, 1/|q_i| joins this lane's scale
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)qf[kk][e], (float)qf[kk][e], ss);
    sl2 *= rsqrtf(half_swap_sum(ss));
  }
  if (p.opt.gate_w != nullptr && p.mode == kModePi) {   // alpha = sigmoid(<w_h, q_i> + b_h)
    const int hg = (p.opt.gate_bh0 + bh) % p.opt.gate_hq;
    const float *w = p.opt.gate_w + (size_t)hg * D + 8 * h;
    f32x4 wv[NQF][2];
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk) {
      wv[kk][0] = *(const f32x4 *)(w + 16 * kk);
      wv[kk][1] = *(const f32x4 *)(w + 16 * kk + 4);
    }
    float z = 0.f;
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) z = fmaf((float)qf[kk][e], wv[kk][e >> 2][e & 3], z);
    bias = log2_sigmoid(half_swap_sum(z) + p.opt.gate_b[hg]);
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;

  // Seed with the skip-key partial state (pi-Attention union, one softmax).
  if (p.skip_ml != nullptr && qvalid && qi >= p.skip_first) {
    const size_t row = (size_t)bh * N + qi;
    const float2 ml = *(const float2 *)(p.skip_ml + 2 * row);
    m_run = ml.x;
    if (h == 0) l_run = ml.y;
    const bf16 *ap = (const bf16 *)p.skip_acc + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        // 16-byte loads, back to the accumulator layout (half h: 4h..4h+3 of each 8)
        uint2 pk[2];
        half_ungroup(*(const uint4 *)(ap + 32 * db + 16 * jp + 8 * h), pk[0], pk[1]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int j4 = 2 * jp + j;
          acc[db][4 * j4 + 0] = __uint_as_float(pk[j].x << 16);
          acc[db][4 * j4 + 1] = __uint_as_float(pk[j].x & 0xffff0000u);
          acc[db][4 * j4 + 2] = __uint_as_float(pk[j].y << 16);
          acc[db][4 * j4 + 3] = __uint_as_float(pk[j].y & 0xffff0000u);
        }
      }
  }

  // ---- per-wave key range ------------------------------------------------
  const int hi_i = key_hi(qi, N, p.mode, p.k_win, p.seg);
  const bool wave_live = q0 < N;
  const int w_hi = key_hi(min(q0 + 31, N - 1), N, p.mode, p.k_win, p.seg);
  const int w_hi_first = key_hi(min(q0, N - 1), N, p.mode, p.k_win, p.seg);   // smallest hi of the wave
  const int w_lo = key_lo(min(q0, N - 1), p.mode, p.k_win, p.seg);
  const int w_lo_last = key_lo(min(q0 + 31, N - 1), p.mode, p.k_win, p.seg);
  const bool w_allvalid = q0 + 31 < N;


  // Per-lane LDS byte offsets inside a tile (buffer and key-block offsets are
  // added as constants).  K: row c of a 32-row block, chunk 2kk+h.
  int koff[NQF];
  {
    const int sw = tile_swz<D>(c);
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk) koff[kk] = c * RB + (((2 * kk + h) ^ sw) << 4);
  }
  // V^T fragments: rows 16kk + 4h + tt/4 (+8), bytes 64db + 32(G&1) + 8(tt&3).
  const int G = lane >> 4, tt = lane & 15;
  int voffs[NDB][2];
  {
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      const int r = 4 * h + (tt >> 2) + 8 * sidx;
      const int sw = tile_swz<D>(r);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int byte = 64 * db + 32 * (G & 1) + 8 * (tt & 3);
        voffs[db][sidx] = r * RB + ((((byte >> 4) ^ sw)) << 4) + (byte & 15);
      }
    }
  }

  // Settle every load (q, alpha, skip state and the first tile) here, so no
  // wait for them is placed inside the loop, where it would also stall on the
  // in-flight tile.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Probabilities of a tile are exp2(s * sl2 + bias - m_run) against the
  // running reference m_run (log2 units), rounded to bf16 for the P V
  // product; the row sum adds the same rounded values (v_dot2_f32_bf16 with
  // ones), so numerator and denominator use identical weights.  The first
  // tile a wave computes takes the row max and sets m_run; later tiles skip
  // the max and check instead that each lane's sum of probabilities stays
  // <= 2^8 (so every probability does): only where it does not are the
  // scores recomputed and the max taken, moving m_run up to it.  Either way
  // every probability is at most 2^8 and the result is the same softmax.
  bool fresh = true;   // no tile computed yet by this wave (wave-uniform)
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  auto tile = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int j0 = tile_row(t);
    const bool more = t + 1 < ntiles;
    if (more) stage(tile_row(t + 1), buf ^ 1);   // lands during the compute below

    if (wave_live && j0 <= w_hi && j0 + TBN - 1 >= w_lo) {
      const char *KB = smem + buf * TILE;
      const char *VB = smem + (2 + buf) * TILE;
      // mask cases (wave-uniform): keys above some row's hi / below some row's lo
      const bool hi_part = !w_allvalid || j0 + TBN - 1 > w_hi_first;
      const bool lo_part = !w_allvalid || j0 < w_lo_last;
      f32x16 s[NKB];
      // ---- S^T = K Q^T for the key tile (one 32x32 block per 32 keys), masked ----
      auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          s[kb] = f32x16{};
#pragma unroll
          for (int kk = 0; kk < NQF; ++kk) {
            const bf16x8 a = *(const bf16x8 *)(KB + 32 * kb * RB + koff[kk]);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
          }
        }
        // Issue order: four key-fragment reads ahead of the products, then one
        // read per product (left alone, the compiler keeps two reads in
        // flight and waits on LDS before every other product).
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // 4 LDS reads
#pragma unroll
        for (int i = 0; i < NKB * NQF - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        // key j visible to query i iff lo(i) <= j <= hi(i); tile-local index
        // of register jj of block kb: 32kb + 8(jj/4) + 4h + jj%4
        if (hi_part && lo_part) {
          const int a0 = lo_i - j0 - 4 * h, span = hi_i - lo_i;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
              const int off = 32 * kb + 8 * (jj >> 2) + (jj & 3);
              if ((unsigned)(off - a0) > (unsigned)span) s[kb][jj] = -INFINITY;
            }
        } else if (hi_part) {
          const int th = hi_i - j0 - 4 * h;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
              if (32 * kb + 8 * (jj >> 2) + (jj & 3) > th) s[kb][jj] = -INFINITY;
        } else if (lo_part) {
          const int tl = lo_i - j0 - 4 * h;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
              if (32 * kb + 8 * (jj >> 2) + (jj & 3) < tl) s[kb][jj] = -INFINITY;
        }
      };
      bf16x8 pb[2 * NKB];
      float lsum;
      auto probs = [&](float nb) __attribute__((always_inline)) {
        lsum = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2 * NKB; ++kk) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(s[kk >> 1][8 * (kk & 1) + 2 * e], sl2, nb));
            const float p1 = fast_exp2(fmaf(s[kk >> 1][8 * (kk & 1) + 2 * e + 1], sl2, nb));
            const bf16x2 pr = {(bf16)p0, (bf16)p1};
            w[e] = __builtin_bit_cast(unsigned, pr);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
          }
          pb[kk] = __builtin_bit_cast(bf16x8, w);
        }
      };

      // Row max, m_run moved up to it, probabilities against it.
      auto with_max = [&]() __attribute__((always_inline)) {
        float mx = s[0][0];
#pragma unroll
        for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, s[0][jj]);
#pragma unroll
        for (int kb = 1; kb < NKB; ++kb)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s[kb][jj]);
        mx = half_swap_max(mx);
        const float m_new = mx * sl2 + bias;
        if (__any(m_new > m_run)) {
          const float mr = fmaxf(m_run, m_new);
          const float f = fast_exp2(m_run - mr);
          l_run *= f;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db] *= f;
          m_run = mr;
        }
        probs(bias - m_run);
      };

      scores();
      if (fresh) {
        with_max();
        fresh = false;
      } else {
        probs(bias - m_run);
        if (__any(!(lsum <= kSumCap))) {
          // The probabilities replaced the scores: recompute them from the
          // tile still in LDS (the empty asm makes the compiler re-read it
          // rather than hold the first reads' fragments in registers).
          asm volatile("" ::: "memory");
          scores();
          with_max();
        }
      }
      l_run += lsum;

      // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
      for (int kk = 0; kk < 2 * NKB; ++kk) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char *base = VB + 16 * kk * RB;
          const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(base + voffs[db][0]));
          const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(base + voffs[db][1]));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(lo, hi), pb[kk], acc[db], 0, 0, 0);
        }
      }
      // the same for the value fragments: four products' reads ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 2 * NKB * NDB - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }

    if (more) wait_dma();
    __syncthreads();
  };
  // Two tiles per trip, so each copy's LDS buffer offsets are constants.
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = acc / l ---------------------------------------------
  const float l_tot = half_swap_sum(l_run);
  if (!qvalid) return;
  // Row normaliser (natural log): scores are carried in log2 units.
  if (p.lse != nullptr && h == 0) p.lse[(size_t)bh * N + qi] = (m_run + __log2f(l_tot)) * kLn2;
  const float inv = 1.0f / l_tot;
  bf16 *op = (bf16 *)p.o + ((size_t)bh * N + qi) * D;
  const bf16 *gp = p.opt.out_gate != nullptr ? (const bf16 *)p.opt.out_gate + ((size_t)bh * N + qi) * D : nullptr;
  // The wave half once more, from the lane count: a copy of h kept from
  // before the tile walk held a register through it (at d = 64 the register
  // that keeps four waves per SIMD).
  const int hs = (int)(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5);
  // Output gate rows, all loaded (16 bytes per lane) before any is used.
  uint4 gq[NDB][2];
  if (gp != nullptr) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) gq[db][jp] = *(const uint4 *)(gp + 32 * db + 16 * jp + 8 * hs);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      uint2 gk[2];
      if (gp != nullptr) half_ungroup(gq[db][jp], gk[0], gk[1]);   // back to the accumulator layout
      uint2 pk[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int j4 = 2 * jp + j;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * j4 + e] * inv;
        if (gp != nullptr) {   // output gate o * sigmoid(g)
          x[0] *= sigmoidf_fast(__uint_as_float(gk[j].x << 16));
          x[1] *= sigmoidf_fast(__uint_as_float(gk[j].x & 0xffff0000u));
          x[2] *= sigmoidf_fast(__uint_as_float(gk[j].y << 16));
          x[3] *= sigmoidf_fast(__uint_as_float(gk[j].y & 0xffff0000u));
        }
        pk[j] = pack_bf16x4(x[0], x[1], x[2], x[3]);
      }
      // 16-byte stores: half hs writes elements 16 jp + 8 hs .. +7 of the 32-block
      *(uint4 *)(op + 32 * db + 16 * jp + 8 * hs) = half_regroup(pk[0], pk[1]);
    }
}

template <typename T, int D>
hipError_t launch_t(const PrefillArgs &a, hipStream_t s) {
  Params p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.alpha = a.alpha; p.o = a.o;
  p.skip_ml = a.skip_ml; p.skip_acc = a.skip_acc; p.lse = a.lse;
  p.N = a.N; p.Hq = a.Hq; p.Hkv = a.Hkv; p.mode = a.mode; p.k_win = a.k_win; p.seg = a.seg;
  p.nqb = (a.N + BM - 1) / BM;
  p.total = a.B * a.Hq * p.nqb;
  p.skip_first = a.skip_first;
  // Rank order pays where block costs vary a lot (ECP, near-dense causal
  // windows); narrow windows cost the same per block and keep head order.
  const int BH = a.B * a.Hq;
  const bool uneven = a.mode == kModeEcp || (long long)a.k_win * 4 >= a.N;
  p.heads_per_xcd = (uneven && BH % 8 == 0) ? BH / 8 : 0;
  // Heads of one rank walk: as many as keep their K and V within about 3 MB
  // (the XCD's L2 is 4 MB), and a divisor of heads_per_xcd.  Walking all of an
  // XCD's heads at once balances slightly better but re-reads K/V from HBM
  // (measured 2.1x the algorithmic fetch for ECP, against 0.96x with groups).
  p.rank_group = 1;
  if (p.heads_per_xcd > 0) {
    const long long kv_head = 2LL * a.N * D * (long long)sizeof(T) / (a.Hq / a.Hkv);  // K+V share per query head
    for (int gsz = p.heads_per_xcd; gsz >= 1; --gsz)
      if (p.heads_per_xcd % gsz == 0 && gsz * kv_head <= (3LL << 20)) {
        p.rank_group = gsz;
        break;
      }
  }
  p.ecp_J = p.ecp_C = 0;
  if (a.mode == kModeEcp && a.seg % BM == 0 && a.N % a.seg == 0) {
    p.ecp_J = a.seg / BM;
    p.ecp_C = a.N / a.seg;
  }
  p.opt = a.opt;
  p.scale_log2 = kLog2e * (a.opt.score_scale > 0.f ? a.opt.score_scale : 1.0f / sqrtf((float)D));
  // d = 128 uses 32-key tiles: 167 VGPRs and 32 KB of LDS let three waves
  // share each SIMD (64-key tiles: 212 VGPRs, 64 KB, two waves), which more
  // than pays for the doubled per-tile overhead.
  if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((prefill_bf16_kernel<D, D == 64 ? 64 : 32>), dim3(p.total), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3(p.total), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Gate network pre-pass: alpha of every query row from the two-layer gate
// network (pi-Attention section 2 item 3), computed once and written to the
// workspace, where the skip pass and the prefill take it as their alpha
// input.  A wave takes kGateBlocks blocks of 32 rows of one (batch, head) in
// the prefill's lane layout: the first layer's rows are loaded and split into
// bf16 parts once, and each block is one matrix product on its query
// fragments (gate_mlp_logit_32).  alpha is clamped to [FLT_MIN, 1]: a logit
// below about -87 would otherwise give alpha = 0 (a -inf local prior).
constexpr int kGateBlocks = 8;

template <typename T, int D>
__global__ __launch_bounds__(256) void gate_alpha_kernel(const T *q, float *alpha, int BH, int N, int Hq, int nwb,
                                                         FusedOpts opt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int gw = blockIdx.x * 4 + wave;           // global wave: (batch, head) and its range of row blocks
  const int bh = gw / nwb, wb = gw % nwb;
  if (bh >= BH) return;                           // the grid's last workgroup may hold spare waves (no barriers)
  const GateMlp gm = make_gate(opt.gate_w, opt.gate_b, opt.gate_w2, opt.gate_b2, opt.gate_hidden, bh % Hq, D);
  if constexpr (sizeof(T) == 2) {
    const GateRows32<D> rows = gate_rows_32<D>(gm, lane);
#pragma unroll 2
    for (int blk = 0; blk < kGateBlocks; ++blk) {
      const int qi = (wb * kGateBlocks + blk) * 32 + c;
      if ((wb * kGateBlocks + blk) * 32 >= N) break;   // wave-uniform
      const T *row = q + ((size_t)bh * N + (qi < N ? qi : N - 1)) * D;
      bf16x8 qf[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8 *)(row + 16 * kk + 8 * h);
      const float z = gate_mlp_logit_32<D>(qf, rows, gm, lane);
      if (qi < N && h == 0) alpha[(size_t)bh * N + qi] = fmaxf(1.0f / (1.0f + __expf(-z)), 1.17549435e-38f);
    }
  } else {
    for (int blk = 0; blk < kGateBlocks; ++blk) {
      const int qi = (wb * kGateBlocks + blk) * 32 + c;
      if ((wb * kGateBlocks + blk) * 32 >= N) break;   // wave-uniform
      const T *row = q + ((size_t)bh * N + (qi < N ? qi : N - 1)) * D;
      float qf[D / 2];
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) qf[kk] = row[2 * kk + h];
      const float z = gate_mlp_logit_32_f32<D>(qf, gm, lane);
      if (qi < N && h == 0) alpha[(size_t)bh * N + qi] = fmaxf(1.0f / (1.0f + __expf(-z)), 1.17549435e-38f);
    }
  }
}

hipError_t launch_gate_alpha(const void *q, float *alpha, int BH, int Hq, int N, int d, int dtype, const FusedOpts &o,
                             hipStream_t s) {
  const int nwb = (N + 32 * kGateBlocks - 1) / (32 * kGateBlocks);   // waves per (batch, head)
  const long long waves = (long long)BH * nwb;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (dtype == kBF16) {
    if (d == 64) hipLaunchKernelGGL((gate_alpha_kernel<bf16, 64>), grid, dim3(256), 0, s, (const bf16 *)q, alpha, BH, N, Hq, nwb, o);
    else hipLaunchKernelGGL((gate_alpha_kernel<bf16, 128>), grid, dim3(256), 0, s, (const bf16 *)q, alpha, BH, N, Hq, nwb, o);
  } else {
    if (d == 64) hipLaunchKernelGGL((gate_alpha_kernel<float, 64>), grid, dim3(256), 0, s, (const float *)q, alpha, BH, N, Hq, nwb, o);
    else hipLaunchKernelGGL((gate_alpha_kernel<float, 128>), grid, dim3(256), 0, s, (const float *)q, alpha, BH, N, Hq, nwb, o);
  }
  return hipGetLastError();
}

// L2-normalised copy of key rows (scaled cosine scores): 8 lanes per row,
// 16-byte loads and stores.
template <typename T, int D>
__global__ __launch_bounds__(256) void normalize_rows_kernel(const T *src, T *dst, long long rows) {
  constexpr int L = 8, C = D / L;           // elements per lane
  constexpr int V = 16 / sizeof(T);         // elements per 16-byte chunk
  typedef T vec __attribute__((ext_vector_type(V)));
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = tid / L;
  const int part = (int)(tid % L);
  const long long r = row < rows ? row : rows - 1;
  const T *sp = src + r * D + part * C;
  vec x[C / V];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < C / V; ++u) {
    x[u] = *(const vec *)(sp + u * V);
#pragma unroll
    for (int e = 0; e < V; ++e) ss = fmaf(to_f32<T>(x[u][e]), to_f32<T>(x[u][e]), ss);
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  const float inv = rsqrtf(ss);
  if (row >= rows) return;
  T *dp = dst + r * D + part * C;
#pragma unroll
  for (int u = 0; u < C / V; ++u) {
    vec y;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      if constexpr (sizeof(T) == 2) y[e] = __builtin_bit_cast(bf16, f32_to_bf16_bits(to_f32<T>(x[u][e]) * inv));
      else y[e] = x[u][e] * inv;
    }
    *(vec *)(dp + u * V) = y;
  }
}

hipError_t launch_normalize_rows(const void *src, void *dst, long long rows, int d, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)((rows * 8 + 255) / 256));
  if (dtype == kBF16) {
    if (d == 64) hipLaunchKernelGGL((normalize_rows_kernel<bf16, 64>), grid, dim3(256), 0, s, (const bf16 *)src, (bf16 *)dst, rows);
    else hipLaunchKernelGGL((normalize_rows_kernel<bf16, 128>), grid, dim3(256), 0, s, (const bf16 *)src, (bf16 *)dst, rows);
  } else {
    if (d == 64) hipLaunchKernelGGL((normalize_rows_kernel<float, 64>), grid, dim3(256), 0, s, (const float *)src, (float *)dst, rows);
    else hipLaunchKernelGGL((normalize_rows_kernel<float, 128>), grid, dim3(256), 0, s, (const float *)src, (float *)dst, rows);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  if (a.dtype == kBF16) return a.d == 64 ? launch_t<bf16, 64>(a, s) : launch_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_t<float, 64>(a, s) : launch_t<float, 128>(a, s);
}

}  // namespace sa
