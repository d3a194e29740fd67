// backward.hip -- backward pass of the structured-sparse attention (bf16 I/O,
// fp32 accumulation) for gfx950.
//
// Gradients of a scalar loss given dO, by the chain rule through the forward
// (one softmax over each query's key set with the gate as a log-prior,
// pi-Attention section 2 items 1-3; ECP section 2; LT2 section 2.1):
//   P_ij = exp(score_ij - lse_i),  dP_ij = <dO_i, v_j>,  D_i = <dO_i, o_i>
//   dS_ij = P_ij (dP_ij - D_i)
//   dq_i = sum_j dS_ij k_j / sqrt(d),  dk_j = sum_i dS_ij q_i / sqrt(d),
//   dv_j = sum_i P_ij dO_i,
//   dalpha_i = sum_{j local} dS_ij / alpha_i - sum_{j skip} dS_ij / (1 - alpha_i).
// lse comes from the training forward (sparse_attn_fwd_lse).
// The gate gradient is taken in an equivalent form: sum_j dS_ij = 0 for every
// row (sum_j P_ij dP_ij = <dO_i, o_i> = D_i), so
//   dalpha_i = -sum_{j skip} dS_ij / (alpha_i (1 - alpha_i))
//            = -sum_{j skip} exp(score0_ij - lse_i) (dP_ij - D_i) / alpha_i,
// with score0 the score without the prior.  The direct form divides the
// window sum, which is minus the (small) skip sum plus the rounding error of
// D_i from the bf16 forward output, by alpha_i; this form has no such
// cancellation, is exactly 0 on rows without skip keys and is finite at
// alpha_i = 1.
//
// Kernels (one call runs them in this order):
//   bwd_prep_kernel   D_i and c_i = log2(prior of local keys) - lse_i*log2(e)
//   skip_bwd_q_kernel / skip_bwd_kv_kernel   (pi-Attention with skip keys)
//       the skip-key contributions to dq (query-owned; also writes dalpha)
//       and dk, dv (key-owned), fp32, written to the workspace; VALU dot
//       products over the <= M skip keys of each row
//   bwd_dq_kernel     query-stationary over the window / ECP keys: the
//       forward's tile walk with S^T = K Q^T and dP^T = V dO^T on the matrix
//       cores, dS, then dQ^T += K^T dS^T (K^T fragments by transposed LDS
//       reads); adds the skip seed and writes dq (bf16) (and dalpha = 0 when
//       no row has a skip key)
//   bwd_dkv_kernel    key-stationary: a workgroup keeps 128 keys (K and V as
//       MFMA operands in registers) and walks the query tiles that attend
//       them, for every query head of the GQA group: S = Q K^T, dP = dO V^T,
//       dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by transposed LDS reads);
//       adds the skip seed and writes dk, dv (bf16)
// Q/dO and K/V tiles are staged with the direct-to-LDS loads and row swizzle
// of the forward.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr int BN = 64;     // rows of a staged tile
constexpr int BM = 128;    // rows (queries or keys) a workgroup owns

struct Params {
  const bf16 *q, *k, *v, *o, *dO;
  const float *alpha, *lse;
  bf16 *dq, *dk, *dv;
  float *dalpha;
  float *Dv, *cv;                       // [B*Hq*N]
  float *dq_s, *dk_s, *dv_s;            // skip contributions (nullptr without skips)
  int B, Hq, Hkv, N, mode, k_win, pi, M, m_min, seg, grp;
  int nqb, nkb;
  float scale_log2, scale;
};

// ---- D_i = <dO_i, o_i>,  c_i = log2(alpha_i) - lse_i log2(e) -----------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(Params p, long long rows) {
  constexpr int L = 8;                              // lanes per row
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = tid / L;
  const int part = (int)(tid % L);
  float acc = 0.f;
  if (row < rows) {
    const bf16 *a = p.dO + row * D + part * (D / L);
    const bf16 *b = p.o + row * D + part * (D / L);
#pragma unroll
    for (int c = 0; c < D / L; c += 8) {
      const bf16x8 x = *(const bf16x8 *)(a + c), y = *(const bf16x8 *)(b + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (row < rows && part == 0) {
    p.Dv[row] = acc;
    float c = -p.lse[row] * kLog2e;
    if (p.mode == kModePi && p.alpha != nullptr) c += __log2f(p.alpha[row]);
    p.cv[row] = c;
  }
}

// ---- skip keys, query-owned: dq's skip term and the gate gradient -------------
// 8 lanes per query row, D/8 dims each.  Writes every row (zeros without skips).
template <int D>
__global__ __launch_bounds__(256) void skip_bwd_q_kernel(Params p, long long rows) {
  constexpr int L = 8, C = D / L;
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = tid / L;
  const int part = (int)(tid % L);
  const bool live = row < rows;
  const long long r = live ? row : 0;
  const int i = (int)(r % p.N);
  const long long bh = r / p.N;
  const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq), g = h / p.grp;
  const bf16 *kb = p.k + (size_t)(b * p.Hkv + g) * p.N * D + part * C;
  const bf16 *vb = p.v + (size_t)(b * p.Hkv + g) * p.N * D + part * C;
  float qv[C], dov[C], dq[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    qv[c] = (float)p.q[r * D + part * C + c];
    dov[c] = (float)p.dO[r * D + part * C + c];
    dq[c] = 0.f;
  }
  const float lse = p.lse[r], Dd = p.Dv[r];
  const float a = p.alpha != nullptr ? p.alpha[r] : 1.f;
  float da = 0.f;
  // Skip keys i - m*pi, m = m_min..M, >= 0 (the same number on all 8 lanes).
  const int mmax = (i - p.m_min * p.pi) >= 0 ? min(p.M, i / p.pi) : p.m_min - 1;
  for (int m = p.m_min; m <= mmax; ++m) {
    const int j = i - m * p.pi;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      s = fmaf(qv[c], (float)kb[(size_t)j * D + c], s);
      dp = fmaf(dov[c], (float)vb[(size_t)j * D + c], dp);
    }
#pragma unroll
    for (int w = 1; w < L; w <<= 1) {
      s += __shfl_xor(s, w, 64);
      dp += __shfl_xor(dp, w, 64);
    }
    const float s0 = s * p.scale;                     // score without the prior
    const float pnp = __expf(s0 - lse);               // P_ij / (1 - alpha_i)
    const float ds = pnp * (1.0f - a) * (dp - Dd);    // dS_ij
    da -= pnp * (dp - Dd);
#pragma unroll
    for (int c = 0; c < C; ++c) dq[c] = fmaf(ds * p.scale, (float)kb[(size_t)j * D + c], dq[c]);
  }
  if (!live) return;
#pragma unroll
  for (int c = 0; c < C; ++c) p.dq_s[r * D + part * C + c] = dq[c];
  if (part == 0 && p.dalpha != nullptr) p.dalpha[r] = da / a;
}

// ---- skip keys, key-owned: dk and dv ------------------------------------------
// 8 lanes per key row of [B, Hkv, N]; loops over the GQA group's heads and the
// queries j + m*pi that have key j as a skip key.  Writes every key row.
template <int D>
__global__ __launch_bounds__(256) void skip_bwd_kv_kernel(Params p, long long kvrows) {
  constexpr int L = 8, C = D / L;
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = tid / L;
  const int part = (int)(tid % L);
  const bool live = row < kvrows;
  const long long r = live ? row : 0;
  const int j = (int)(r % p.N);
  const long long bg = r / p.N;
  const int b = (int)(bg / p.Hkv), g = (int)(bg % p.Hkv);
  float kv[C], vv[C], dk[C], dv[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    kv[c] = (float)p.k[r * D + part * C + c];
    vv[c] = (float)p.v[r * D + part * C + c];
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  for (int hh = 0; hh < p.grp; ++hh) {
    const size_t qrow0 = ((size_t)b * p.Hq + g * p.grp + hh) * p.N;
    for (int m = p.m_min; m <= p.M; ++m) {
      const long long il = (long long)j + (long long)m * p.pi;
      if (il >= p.N) break;
      const size_t qr = qrow0 + (size_t)il;
      const bf16 *qp = p.q + qr * D + part * C, *dop = p.dO + qr * D + part * C;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        s = fmaf((float)qp[c], kv[c], s);
        dp = fmaf((float)dop[c], vv[c], dp);
      }
#pragma unroll
      for (int w = 1; w < L; w <<= 1) {
        s += __shfl_xor(s, w, 64);
        dp += __shfl_xor(dp, w, 64);
      }
      const float a = p.alpha != nullptr ? p.alpha[qr] : 1.f;
      const float P = __expf(s * p.scale - p.lse[qr]) * (1.0f - a);
      const float ds = P * (dp - p.Dv[qr]);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        dk[c] = fmaf(ds * p.scale, (float)qp[c], dk[c]);
        dv[c] = fmaf(P, (float)dop[c], dv[c]);
      }
    }
  }
  if (!live) return;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    p.dk_s[r * D + part * C + c] = dk[c];
    p.dv_s[r * D + part * C + c] = dv[c];
  }
}

// Store 16 accumulator values of a 32x32 C tile (rows 8(j/4) + 4h + j%4 of the
// 32-row block db, column = this lane) as bf16, scaled, plus an fp32 seed.
template <int D>
__device__ __forceinline__ void store_rows_bf16(bf16 *dst, const f32x16 (&acc)[D / 32], float scale,
                                                const float *seed, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int dim = 32 * db + 8 * j4 + 4 * h;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * j4 + e] * scale;
      if (seed != nullptr) {
        const f32x4 sd = *(const f32x4 *)(seed + dim);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] += sd[e];
      }
      ushort4 u;
      u.x = f32_to_bf16_bits(x[0]);
      u.y = f32_to_bf16_bits(x[1]);
      u.z = f32_to_bf16_bits(x[2]);
      u.w = f32_to_bf16_bits(x[3]);
      *(ushort4 *)(dst + dim) = u;
    }
}

// Per-lane LDS byte offsets of MFMA row fragments (row c of a 32-row block,
// chunk 2kk+h) and of transposed fragments (rows 16kk + 4h + tt/4 (+8),
// bytes 64db + 32(G&1) + 8(tt&3)) in a swizzled 64-row tile.
template <int D>
struct TileOffsets {
  int row[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ TileOffsets(int lane) {
    constexpr int RB = D * 2;
    const int h = lane >> 5, c = lane & 31, G = lane >> 4, tt = lane & 15;
    const int sw = tile_swz<D>(c);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) row[kk] = c * RB + (((2 * kk + h) ^ sw) << 4);
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx) {
      const int r = 4 * h + (tt >> 2) + 8 * sidx;
      const int sr = tile_swz<D>(r);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int byte = 64 * db + 32 * (G & 1) + 8 * (tt & 3);
        tr[db][sidx] = r * RB + (((byte >> 4) ^ sr) << 4) + (byte & 15);
      }
    }
  }
};

// Stage rows [j0, j0+64) of a [rows, D] bf16 matrix into a swizzled LDS tile
// with the workgroup's 4 waves (rows past `last` re-read row `last`).
template <int D>
__device__ __forceinline__ void stage_tile(const bf16 *src, int j0, int last, unsigned dst, int wave, int lane) {
  constexpr int CPR = D / 8, PER_WAVE = BN * D * 2 / 1024 / 4;
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int slot = PER_WAVE * wave + u;
    const int pch = 64 * slot + lane;
    const int row = pch / CPR;
    const int chunk = (pch % CPR) ^ tile_swz<D>(row);
    const int key = min(j0 + row, last);
    dma16(src, (unsigned)((key * D + chunk * 8) * 2), __builtin_amdgcn_readfirstlane(dst + 1024 * slot));
  }
}

// ---- dq and dalpha: query-stationary walk over the window / ECP keys ---------
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(Params p) {
  constexpr int RB = D * 2, TILE = BN * RB, NQF = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];   // K0 K1 V0 V1
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int logical = xcd_remap(blockIdx.x, p.B * p.Hq * p.nqb);
  const int qb = p.nqb - 1 - logical % p.nqb, bh = logical / p.nqb;
  const int hq = bh % p.Hq, b = bh / p.Hq, g = hq / p.grp;
  const int N = p.N;
  const int i0 = qb * BM, q0 = i0 + wave * 32, qi = q0 + c;
  const bool qvalid = qi < N;
  const size_t row = (size_t)bh * N + (qvalid ? qi : 0);
  const bf16 *Kp = p.k + (size_t)(b * p.Hkv + g) * N * D;
  const bf16 *Vp = p.v + (size_t)(b * p.Hkv + g) * N * D;

  bf16x8 qf[NQF], df[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) {
    qf[kk] = qvalid ? *(const bf16x8 *)(p.q + row * D + 16 * kk + 8 * h) : bf16x8{};
    df[kk] = qvalid ? *(const bf16x8 *)(p.dO + row * D + 16 * kk + 8 * h) : bf16x8{};
  }
  const float ci = qvalid ? p.cv[row] : 0.f, Di = qvalid ? p.Dv[row] : 0.f;
  const int lo_i = key_lo(qi, p.mode, p.k_win, p.seg);
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const int hi_wg = min(i0 + BM - 1, N - 1);
  const int t_begin = (key_lo(i0, p.mode, p.k_win, p.seg) / BN) * BN;
  const int ntiles = (hi_wg - t_begin) / BN + 1;
  const bool wave_live = q0 < N;
  const int w_hi = min(q0 + 31, N - 1);
  const int w_lo = key_lo(min(q0, N - 1), p.mode, p.k_win, p.seg);
  const int w_lo_last = key_lo(min(q0 + 31, N - 1), p.mode, p.k_win, p.seg);
  const bool w_allvalid = q0 + 31 < N;
  const TileOffsets<D> off(lane);
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)smem;

  __builtin_amdgcn_s_waitcnt(0);
  stage_tile<D>(Kp, t_begin, N - 1, lds0, wave, lane);
  stage_tile<D>(Vp, t_begin, N - 1, lds0 + 2 * TILE, wave, lane);
  wait_dma();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t_begin + t * BN;
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) {
      stage_tile<D>(Kp, j0 + BN, N - 1, lds0 + (buf ^ 1) * TILE, wave, lane);
      stage_tile<D>(Vp, j0 + BN, N - 1, lds0 + (2 + (buf ^ 1)) * TILE, wave, lane);
    }
    if (wave_live && j0 <= w_hi && j0 + BN - 1 >= w_lo) {
      const char *KB = smem + buf * TILE;
      const char *VB = smem + (2 + buf) * TILE;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NQF; ++kk) {
          const bf16x8 ka = *(const bf16x8 *)(KB + 32 * kb * RB + off.row[kk]);
          const bf16x8 va = *(const bf16x8 *)(VB + 32 * kb * RB + off.row[kk]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[kb], 0, 0, 0);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[kk], dp[kb], 0, 0, 0);
        }
      }
      const bool full = w_allvalid && (j0 + BN - 1 <= q0) && (j0 >= w_lo_last);
      const int a0 = lo_i - j0 - 4 * h, span = qi - lo_i;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int o = 32 * kb + 8 * (jj >> 2) + (jj & 3);
          float pr = fast_exp2(fmaf(s[kb][jj], p.scale_log2, ci));
          if (!full && (unsigned)(o - a0) > (unsigned)span) pr = 0.f;
          s[kb][jj] = pr * (dp[kb][jj] - Di);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb[e] = (bf16)s[kk >> 1][8 * (kk & 1) + e];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char *base = KB + 16 * kk * RB;
          const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(base + off.tr[db][0]));
          const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(base + off.tr[db][1]));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(lo, hi), sb, acc[db], 0, 0, 0);
        }
      }
    }
    if (more) wait_dma();
    __syncthreads();
  }
  if (!qvalid) return;
  store_rows_bf16<D>(p.dq + row * D, acc, p.scale, p.dq_s != nullptr ? p.dq_s + row * D : nullptr, h);
  if (p.dalpha != nullptr && p.dq_s == nullptr && h == 0) p.dalpha[row] = 0.f;
}

// Last query position that has key j in its window / ECP range (at most N - 1).
__device__ __forceinline__ int last_query(int j, const Params &p) {
  const long long last = p.mode == kModeEcp ? ((long long)(j / p.seg) + 2) * p.seg - 1 : (long long)j + p.k_win;
  return last < p.N - 1 ? (int)last : p.N - 1;
}

// ---- dk and dv: key-stationary walk over the query tiles -------------------------
// d = 128 holds K, V (64 VGPRs) and the dK, dV accumulators (128) per lane:
// one wave per SIMD, with the 512-entry register budget that allows.
template <int D>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkv_kernel(Params p) {
  constexpr int RB = D * 2, TILE = BN * RB, NQF = D / 16, NDB = D / 32;
  // Q0 Q1 dO0 dO1 tiles, then per-query c and D (two buffers of 64 floats each)
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE + 4 * 256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int logical = xcd_remap(blockIdx.x, p.B * p.Hkv * p.nkb);
  const int kb0 = logical % p.nkb, bg = logical / p.nkb;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int N = p.N;
  const int k0 = kb0 * BM, j_w = k0 + wave * 32, kj = j_w + c;
  const bool kvalid = kj < N;
  const size_t krow = (size_t)bg * N + (kvalid ? kj : 0);

  bf16x8 kf[NQF], vf[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) {
    kf[kk] = kvalid ? *(const bf16x8 *)(p.k + krow * D + 16 * kk + 8 * h) : bf16x8{};
    vf[kk] = kvalid ? *(const bf16x8 *)(p.v + krow * D + 16 * kk + 8 * h) : bf16x8{};
  }
  f32x16 adk[NDB], adv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    adk[db] = f32x16{};
    adv[db] = f32x16{};
  }
  const int kw_last = min(j_w + 31, N - 1);
  const bool wave_live = j_w < N;
  const int hi_q = last_query(min(k0 + BM - 1, N - 1), p);
  const int t_begin = k0;                       // the first query that can see key k0 is k0
  const int ntiles = (hi_q - t_begin) / BN + 1;
  const int wq_hi = last_query(kw_last, p);   // last query seeing this wave's keys
  const int w_lq_first = last_query(min(j_w, N - 1), p);   // last query seeing all of them
  const bool w_allvalid = j_w + 31 < N;
  // Query iq sees key kj iff kj <= iq <= last_query(kj) (key_lo is
  // non-decreasing in iq); an invalid key gets an empty range.
  const int vis_lo = kvalid ? kj : -(1 << 30);
  const unsigned vis_span = kvalid ? (unsigned)(last_query(kj, p) - kj) : 0u;
  const TileOffsets<D> off(lane);
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
  const float *cl = (const float *)(smem + 4 * TILE);       // [2][64] c, then [2][64] D

  auto stage_vec = [&](const float *src, int i0v, unsigned dst) __attribute__((always_inline)) {
    // 64 floats, one per lane of wave 0 (entries past N re-read entry N - 1)
    if (wave == 0) dma4(src, (unsigned)(min(i0v + lane, N - 1) * 4), __builtin_amdgcn_readfirstlane(dst));
  };

  __builtin_amdgcn_s_waitcnt(0);
  for (int hh = 0; hh < p.grp; ++hh) {
    const size_t qbase = ((size_t)b * p.Hq + g * p.grp + hh) * N;
    const bf16 *Qp = p.q + qbase * D, *Op = p.dO + qbase * D;
    const float *Cp = p.cv + qbase, *Dp = p.Dv + qbase;
    stage_tile<D>(Qp, t_begin, N - 1, lds0, wave, lane);
    stage_tile<D>(Op, t_begin, N - 1, lds0 + 2 * TILE, wave, lane);
    stage_vec(Cp, t_begin, lds0 + 4 * TILE);
    stage_vec(Dp, t_begin, lds0 + 4 * TILE + 512);
    wait_dma();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int i0 = t_begin + t * BN;
      const int buf = t & 1;
      const bool more = t + 1 < ntiles;
      if (more) {
        stage_tile<D>(Qp, i0 + BN, N - 1, lds0 + (buf ^ 1) * TILE, wave, lane);
        stage_tile<D>(Op, i0 + BN, N - 1, lds0 + (2 + (buf ^ 1)) * TILE, wave, lane);
        stage_vec(Cp, i0 + BN, lds0 + 4 * TILE + 256 * (buf ^ 1));
        stage_vec(Dp, i0 + BN, lds0 + 4 * TILE + 512 + 256 * (buf ^ 1));
      }
      // this wave's keys [j_w, kw_last] are seen by queries [j_w, wq_hi]
      if (wave_live && i0 + BN - 1 >= j_w && i0 <= wq_hi) {
        const char *QB = smem + buf * TILE;
        const char *OB = smem + (2 + buf) * TILE;
        const float *cq = cl + 64 * buf, *dq = cl + 128 + 64 * buf;
        // every (query, key) of the tile visible: no per-element mask
        const bool full = w_allvalid && i0 >= kw_last && i0 + BN - 1 <= w_lq_first;
        // The 64 queries in two halves of 32 (fewer live accumulators).
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2) {
          f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int kk = 0; kk < NQF; ++kk) {
            const bf16x8 qa = *(const bf16x8 *)(QB + 32 * qb2 * RB + off.row[kk]);
            const bf16x8 oa = *(const bf16x8 *)(OB + 32 * qb2 * RB + off.row[kk]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kk], dp, 0, 0, 0);
          }
          // element jj: query i0 + 32 qb2 + 8(jj/4) + 4h + jj%4, key kj
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int ql = 32 * qb2 + 8 * j4 + 4 * h;        // tile-local query of element 4 j4
            const f32x4 cvv = *(const f32x4 *)(cq + ql);
            const f32x4 dvv = *(const f32x4 *)(dq + ql);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int jj = 4 * j4 + e;
              float pr = fast_exp2(fmaf(s[jj], p.scale_log2, cvv[e]));
              if (!full && (unsigned)(i0 + ql + e - vis_lo) > vis_span) pr = 0.f;
              s[jj] = pr;
              dp[jj] = pr * (dp[jj] - dvv[e]);
            }
          }
          // dV^T += dO^T P, dK^T += Q^T dS over these 32 queries
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int kk = 2 * qb2 + k2;
            bf16x8 pb, sb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pb[e] = (bf16)s[8 * k2 + e];
              sb[e] = (bf16)dp[8 * k2 + e];
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const char *ob = OB + 16 * kk * RB, *qbp = QB + 16 * kk * RB;
              const short4v olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(ob + off.tr[db][0]));
              const short4v ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(ob + off.tr[db][1]));
              const short4v qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(qbp + off.tr[db][0]));
              const short4v qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(qbp + off.tr[db][1]));
              adv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(olo, ohi), pb, adv[db], 0, 0, 0);
              adk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(qlo, qhi), sb, adk[db], 0, 0, 0);
            }
          }
        }
      }
      if (more) wait_dma();
      __syncthreads();
    }
  }
  if (!kvalid) return;
  store_rows_bf16<D>(p.dk + krow * D, adk, p.scale, p.dk_s != nullptr ? p.dk_s + krow * D : nullptr, h);
  store_rows_bf16<D>(p.dv + krow * D, adv, 1.0f, p.dv_s != nullptr ? p.dv_s + krow * D : nullptr, h);
}

template <int D>
hipError_t launch_t(const BwdArgs &a, hipStream_t s) {
  Params p;
  p.q = (const bf16 *)a.q; p.k = (const bf16 *)a.k; p.v = (const bf16 *)a.v; p.o = (const bf16 *)a.o;
  p.dO = (const bf16 *)a.dO; p.alpha = a.alpha; p.lse = a.lse;
  p.dq = (bf16 *)a.dq; p.dk = (bf16 *)a.dk; p.dv = (bf16 *)a.dv; p.dalpha = a.dalpha;
  p.Dv = a.Dv; p.cv = a.cv; p.dq_s = a.dq_s; p.dk_s = a.dk_s; p.dv_s = a.dv_s;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N; p.mode = a.mode; p.k_win = a.k_win; p.pi = a.pi;
  p.M = a.M; p.m_min = a.m_min; p.seg = a.seg; p.grp = a.Hq / a.Hkv;
  p.nqb = (a.N + BM - 1) / BM;
  p.nkb = (a.N + BM - 1) / BM;
  p.scale = 1.0f / sqrtf((float)D);
  p.scale_log2 = kLog2e * p.scale;
  const long long rows = (long long)a.B * a.Hq * a.N, kvrows = (long long)a.B * a.Hkv * a.N;
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0, s, p, rows);
  if (p.dq_s != nullptr) {
    hipLaunchKernelGGL((skip_bwd_q_kernel<D>), dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0, s, p, rows);
    hipLaunchKernelGGL((skip_bwd_kv_kernel<D>), dim3((unsigned)((kvrows * 8 + 255) / 256)), dim3(256), 0, s, p,
                       kvrows);
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(a.B * a.Hq * p.nqb), dim3(256), 0, s, p);
  hipLaunchKernelGGL((bwd_dkv_kernel<D>), dim3(a.B * a.Hkv * p.nkb), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  return a.d == 64 ? launch_t<64>(a, s) : launch_t<128>(a, s);
}

}  // namespace sa
