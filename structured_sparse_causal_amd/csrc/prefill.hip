// prefill.hip -- window / paired-half-segment attention forward for gfx950.
//
// One workgroup (4 waves) owns a block of 128 consecutive query rows of one
// (batch, head); each wave owns 32 of them.  Key/value tiles of 64 rows stream
// through LDS; the workgroup walks the tiles covering the union of its rows'
// key ranges:
//   window (pi-Attention section 2 item 1; LT2 section 2.1): [max(0,i-k), i]
//   ECP (PAR block, ECP section 2):       [max(0,(floor(i/s)-1)*s), i]
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// every lane then owns ONE query and 32 keys of the tile, so the softmax row
// max and sum are lane-local plus one exchange between the wave halves
// (v_permlane32_swap).  P^T stays in registers as the B operand of
// O^T = V^T P^T; the V^T fragment comes straight from the row-major V tile
// through ds_read_b64_tr_b16.
//
// Pipelining: K/V tiles are double-buffered in LDS.  While a wave computes on
// tile t, the workgroup's global loads of tile t+1 are already in flight into
// registers; they are written to the other LDS buffer after the compute, so
// one barrier per tile suffices and HBM latency hides behind the MFMA work.
//
// The softmax is online in log2 units with lazy rescaling (the running max
// only moves when a tile raises it by more than 8, so exp2 arguments stay
// <= 8): exact, since numerator and denominator use the same reference.
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

struct Params {
  const void *q, *k, *v;
  const float *alpha;
  void *o;
  const float *skip_ml;
  const void *skip_acc;
  int N, Hq, Hkv, mode, k_win, seg, nqb, total, skip_first;
  float scale_log2;
};

__device__ __forceinline__ int key_lo(int i, int mode, int k_win, int seg) {
  if (mode == kModeEcp) {
    const int lo = (i / seg - 1) * seg;
    return lo > 0 ? lo : 0;
  }
  const int lo = i - k_win;
  return lo > 0 ? lo : 0;
}

// LDS tile geometry.  K rows are read as 16-byte MFMA fragments by 32 lanes at
// once (one row each): a 16-byte row pad spreads them over all banks.  V rows
// are read by ds_read_b64_tr_b16 (4 rows x 32 bytes per 16 lanes, two such
// groups 32 bytes apart per half-wave): a row stride of 64 bytes modulo 256
// keeps both groups on disjoint banks.  fp32 tiles use plain 4-byte reads.
template <typename T, int D>
struct Tile {
  static constexpr bool kBF = sizeof(T) == 2;
  static constexpr int LDK = D + (kBF ? 8 : 4);                   // elements
  static constexpr int LDV = kBF ? (D == 64 ? 96 : 160) : D + 4;  // elements
  static constexpr int VEC = 16 / sizeof(T);                       // elements per 16 bytes
  static constexpr int CPR = D / VEC;                              // 16-byte chunks per row
  static constexpr int PER_THREAD = BN * CPR / 256;                // chunks per thread per tensor
  static constexpr int NBUF = kBF ? 2 : 1;
  static constexpr int KSZ = BN * LDK, VSZ = BN * LDV;
};

__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void prefill_kernel(Params p) {
  using TL = Tile<T, D>;
  constexpr bool kBF = TL::kBF;
  constexpr int LDK = TL::LDK, LDV = TL::LDV;
  __shared__ __attribute__((aligned(16))) T Ks[TL::NBUF][TL::KSZ];
  __shared__ __attribute__((aligned(16))) T Vs[TL::NBUF][TL::VSZ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int logical = xcd_remap(blockIdx.x, p.total);
  // Within a head the blocks run last-to-first: late blocks have the longest
  // key ranges (ECP, causal edges), so the light ones form the grid's tail.
  const int qb = p.nqb - 1 - logical % p.nqb, bh = logical / p.nqb;
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int g = hq / (p.Hq / p.Hkv);
  const int N = p.N;
  const int i0 = qb * BM, q0 = i0 + wave * 32, qi = q0 + c;
  const bool qvalid = qi < N;

  const T *Qp = (const T *)p.q + (size_t)bh * N * D;
  const T *Kp = (const T *)p.k + (size_t)(b * p.Hkv + g) * N * D;
  const T *Vp = (const T *)p.v + (size_t)(b * p.Hkv + g) * N * D;

  // ---- per-lane query state --------------------------------------------
  const int lo_i = key_lo(qi, p.mode, p.k_win, p.seg);
  float bias = 0.f;  // log2 of the local prior
  if (p.mode == kModePi && p.alpha != nullptr && qvalid) bias = __log2f(p.alpha[(size_t)bh * N + qi]);

  constexpr int NQF = kBF ? D / 16 : D / 2;
  typedef typename std::conditional<kBF, bf16x8, float>::type QFrag;
  QFrag qf[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) {
    if constexpr (kBF) {
      if (qvalid) qf[kk] = *(const bf16x8 *)(Qp + (size_t)qi * D + 16 * kk + 8 * h);
      else qf[kk] = bf16x8{};
    } else {
      qf[kk] = qvalid ? (float)Qp[(size_t)qi * D + 2 * kk + h] : 0.f;
    }
  }

  constexpr int NDB = D / 32;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;

  // Seed with the skip-key partial state (pi-Attention union, one softmax).
  if (p.skip_ml != nullptr && qvalid && qi >= p.skip_first) {
    const size_t row = (size_t)bh * N + qi;
    m_run = p.skip_ml[2 * row];
    if (h == 0) l_run = p.skip_ml[2 * row + 1];
    const T *ap = (const T *)p.skip_acc + row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const T *src = ap + 32 * db + 8 * j4 + 4 * h;
        if constexpr (kBF) {
          const ushort4 u = *(const ushort4 *)src;
          acc[db][4 * j4 + 0] = bf16_to_f32(u.x);
          acc[db][4 * j4 + 1] = bf16_to_f32(u.y);
          acc[db][4 * j4 + 2] = bf16_to_f32(u.z);
          acc[db][4 * j4 + 3] = bf16_to_f32(u.w);
        } else {
          const f32x4 x = *(const f32x4 *)src;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * j4 + e] = x[e];
        }
      }
  }

  // ---- key-tile range ---------------------------------------------------
  const int hi_wg = min(i0 + BM - 1, N - 1);
  const int t_begin = (key_lo(i0, p.mode, p.k_win, p.seg) / BN) * BN;
  const int ntiles = (hi_wg - t_begin) / BN + 1;
  const bool wave_live = q0 < N;
  const int w_hi = min(q0 + 31, N - 1);
  const int w_lo = key_lo(min(q0, N - 1), p.mode, p.k_win, p.seg);
  const int w_lo_last = key_lo(min(q0 + 31, N - 1), p.mode, p.k_win, p.seg);
  const bool w_allvalid = q0 + 31 < N;
  const float sl2 = p.scale_log2;

  // ---- cooperative staging: global -> registers -> LDS --------------------
  uint4 kreg[TL::PER_THREAD], vreg[TL::PER_THREAD];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int r = 0; r < TL::PER_THREAD; ++r) {
      const int ci = tid + 256 * r;
      const int row = ci / TL::CPR, col = (ci % TL::CPR) * TL::VEC;
      const int key = j0 + row;
      if (key < N) {
        kreg[r] = *(const uint4 *)(Kp + (size_t)key * D + col);
        vreg[r] = *(const uint4 *)(Vp + (size_t)key * D + col);
      } else {
        kreg[r] = make_uint4(0, 0, 0, 0);
        vreg[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < TL::PER_THREAD; ++r) {
      const int ci = tid + 256 * r;
      const int row = ci / TL::CPR, col = (ci % TL::CPR) * TL::VEC;
      *(uint4 *)(&Ks[buf][row * LDK + col]) = kreg[r];
      *(uint4 *)(&Vs[buf][row * LDV + col]) = vreg[r];
    }
  };

  load_tile(t_begin);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t_begin + t * BN;
    const int buf = TL::NBUF == 2 ? (t & 1) : 0;
    const bool more = t + 1 < ntiles;
    if (TL::NBUF == 2 && more) load_tile(j0 + BN);   // in flight during the compute below

    if (wave_live && j0 <= w_hi && j0 + BN - 1 >= w_lo) {
      const T *KB = Ks[buf];
      const T *VB = Vs[buf];
      // ---- S^T = K Q^T for the 64-key tile: two 32x32 blocks -------------------
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const T *krow = KB + (32 * kb + c) * LDK;
#pragma unroll
        for (int kk = 0; kk < NQF; ++kk) {
          if constexpr (kBF) {
            const bf16x8 a = *(const bf16x8 *)(krow + 16 * kk + 8 * h);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
          } else {
            const float a = krow[2 * kk + h];
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[kk], s[kb], 0, 0, 0);
          }
        }
      }

      // ---- mask: key j visible to query i iff lo(i) <= j <= i -----------------
      const bool full = w_allvalid && (j0 + BN - 1 <= q0) && (j0 >= w_lo_last);
      if (!full) {
        // tile-local index of register jj of block kb: 32kb + 8(jj/4) + 4h + jj%4
        const int a0 = lo_i - j0 - 4 * h, span = qi - lo_i;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int off = 32 * kb + 8 * (jj >> 2) + (jj & 3);
            if ((unsigned)(off - a0) > (unsigned)span) s[kb][jj] = -INFINITY;
          }
      }

      // ---- online softmax (log2 units, lazy rescale) ---------------------------
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
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float pv = fast_exp2(fmaf(s[kb][jj], sl2, nb));
          s[kb][jj] = pv;
          lsum += pv;
        }
      l_run += lsum;

      // ---- O^T += V^T P^T ------------------------------------------------------
      if constexpr (kBF) {
        const int G = lane >> 4, tt = lane & 15;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (bf16)s[kk >> 1][8 * (kk & 1) + e];
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int col = 32 * db + 16 * (G & 1) + 4 * (tt & 3);
            const T *r0 = VB + (16 * kk + 4 * h + (tt >> 2)) * LDV + col;
            const T *r1 = r0 + 8 * LDV;
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)r0);
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)r1);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(lo, hi), pb, acc[db], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int tt = 0; tt < 16; ++tt) {
            const T *vrow = VB + (32 * kb + 8 * (tt >> 2) + 4 * h + (tt & 3)) * LDV;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db + c], s[kb][tt], acc[db], 0, 0, 0);
          }
      }
    }

    if (more) {
      if (TL::NBUF == 2) {
        store_tile(buf ^ 1);
      } else {
        __syncthreads();          // single buffer: everyone is done reading it
        load_tile(j0 + BN);
        store_tile(0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: O = acc / l ---------------------------------------------
  const float l_tot = half_swap_sum(l_run);
  if (!qvalid) return;
  const float inv = 1.0f / l_tot;
  T *op = (T *)p.o + ((size_t)bh * N + qi) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int dim = 32 * db + 8 * j4 + 4 * h;
      if constexpr (kBF) {
        ushort4 u;
        u.x = f32_to_bf16_bits(acc[db][4 * j4 + 0] * inv);
        u.y = f32_to_bf16_bits(acc[db][4 * j4 + 1] * inv);
        u.z = f32_to_bf16_bits(acc[db][4 * j4 + 2] * inv);
        u.w = f32_to_bf16_bits(acc[db][4 * j4 + 3] * inv);
        *(ushort4 *)(op + dim) = u;
      } else {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * j4 + e] * inv;
        *(f32x4 *)(op + dim) = x;
      }
    }
}

template <typename T, int D>
hipError_t launch_t(const PrefillArgs &a, hipStream_t s) {
  Params p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.alpha = a.alpha; p.o = a.o;
  p.skip_ml = a.skip_ml; p.skip_acc = a.skip_acc;
  p.N = a.N; p.Hq = a.Hq; p.Hkv = a.Hkv; p.mode = a.mode; p.k_win = a.k_win; p.seg = a.seg;
  p.nqb = (a.N + BM - 1) / BM;
  p.total = a.B * a.Hq * p.nqb;
  p.skip_first = a.skip_first;
  p.scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((prefill_kernel<T, D>), dim3(p.total), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  if (a.dtype == kBF16) return a.d == 64 ? launch_t<bf16, 64>(a, s) : launch_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_t<float, 64>(a, s) : launch_t<float, 128>(a, s);
}

}  // namespace sa
