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
//   bwd_prep_kernel   (output gate only) dO * sigmoid(g), dg, D_i and c_i
//   bwd_dq_kernel     query-stationary over the window / ECP keys: the
//       forward's tile walk with S^T = K Q^T and dP^T = V dO^T on the matrix
//       cores, dS, then dQ^T += K^T dS^T (K^T fragments by transposed LDS
//       reads); writes dq (bf16), dalpha = 0 on rows without skip keys, and
//       (no output gate) D_i = <dO_i, o_i> and c_i = log2(prior of local
//       keys) - lse_i*log2(e) from the rows it holds
//   bwd_dkv_kernel    key-stationary: a workgroup keeps 128 keys (K and V as
//       MFMA operands in registers) and walks the query tiles that attend
//       them, for every query head of the GQA group: S = Q K^T, dP = dO V^T,
//       dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by transposed LDS reads);
//       writes dk, dv (bf16)
//   skip_bwd_kv_kernel / skip_bwd_q_kernel   (pi-Attention with skip keys)
//       the skip-key contributions to dk, dv (key-owned) and dq, dalpha
//       (query-owned), added into the bf16 gradients the walks wrote; 16x16
//       MFMA tiles over the residue chains i mod pi (one kernel when every
//       chain is one tile).  Every row is added by exactly one wave, after
//       the walks (same stream), so no two writers meet.
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
  int skips;                            // pi-Attention with skip keys: the skip kernels run last
  int B, Hq, Hkv, N, mode, k_win, pi, M, m_min, seg, grp;
  int nqb, nkb;
  // skip-key residue chains: periods per residue, first position with a skip
  // key (m_min * pi), query- and key-period tiles per residue, wave counts
  int P, skip_first, nqt, nkt, nwork_q, nwork_kv;
  float scale_log2, scale;
  // output gate y = o * sigmoid(g) (o here is y): the prep pass writes
  // dO * sigmoid(g) to dO_gated, which the other kernels read as dO, and dg
  const bf16 *out_gate;
  bf16 *dgate, *dO_gated;
  // no output gate: the dq kernel forms D_i and c_i itself (it holds the
  // rows of dO already) and writes them for the dk/dv walk and the skip
  // kernels, in place of the prep pass
  int fold_prep;
};

// ---- D_i = <dO_i, o_i>,  c_i = log2(alpha_i) - lse_i log2(e) -----------------
// With an output gate y = o * sigmoid(g) the inputs are dY and y: the
// attention's output gradient is dY * sigmoid(g) (written to dO_gated),
// D_i = <dY_i * sigmoid(g_i), o_i> = <dY_i, y_i>, and dg = dY * y * (1 - sigmoid(g)).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(Params p, long long rows) {
  constexpr int L = 8;                              // lanes per row
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = tid / L;
  const int part = (int)(tid % L);
  float acc = 0.f;
  if (row < rows) {
    const size_t at = (size_t)row * D + part * (D / L);
    const bf16 *a = p.dO + at;
    const bf16 *b = p.o + at;
#pragma unroll
    for (int c = 0; c < D / L; c += 8) {
      const bf16x8 x = *(const bf16x8 *)(a + c), y = *(const bf16x8 *)(b + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
      if (p.out_gate != nullptr) {
        const bf16x8 g = *(const bf16x8 *)(p.out_gate + at + c);
        bf16x8 dog, dg;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-(float)g[e] * kLog2e));
          dog[e] = (bf16)((float)x[e] * sg);
          dg[e] = (bf16)((float)x[e] * (float)y[e] * (1.0f - sg));
        }
        *(bf16x8 *)(p.dO_gated + at + c) = dog;
        *(bf16x8 *)(p.dgate + at + c) = dg;
      }
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

// ---- skip keys: residue chains -------------------------------------------------
// Query i and its skip keys i - m*pi share the residue r = i mod pi; with
// period p = (i - r)/pi, query period p attends key periods p - m for
// m in [m_min, M] (a small dense band per residue, pi-Attention section 2
// item 2).  The 16x16 MFMAs run on tiles of 16 periods of one residue:
//   16x16x32 (K = dims): S = Q K^T and dP = dO V^T (rows queries, columns
//     keys), or with swapped operands S^T, dP^T (rows keys, columns queries);
//   16x16x16 (K = 16 periods): dV^T += dO^T P, dK^T += Q^T dS, dQ^T += K^T dS^T
//     with the transposed operand read from a per-wave LDS copy of the rows
//     the wave holds in registers.
// Skip keys carry the prior log(1 - alpha_i): P = (1 - alpha_i) exp(s - lse_i).
// The gate gradient's skip sum uses exp(s - lse_i) (dP - D_i) directly, so it
// stays finite at alpha_i = 1.

// Transposed 16x16 operand from a wave's LDS rows: lane (G, t) gets
// rows 4G..4G+3 at column c0 + t.
template <int LD>
__device__ __forceinline__ bf16x4 lds_tr16(const bf16 *rows, int c0, int G, int t) {
  const bf16 *src = rows + (4 * G + (t >> 2)) * LD + c0 + 4 * (t & 3);
  return as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)src));
}

// Gradient rows added back with 16-byte accesses: a 16 x D block in the 16x16
// MFMA C layout (lane (G, t) holds values 16db + 4G + e of row t) is written
// to the wave's LDS as fp32 rows of stride D + 4 floats, then each lane takes
// the chunks 32kk + 8G .. +7 of row t (the layout of the operand loads), adds
// the bf16 values read from the destination earlier in that layout, and
// stores the sum rounded to bf16 once.  Callers order the LDS accesses
// (wave_lds_sync) around stage_rows.
template <int D>
__device__ __forceinline__ void stage_rows(float *buf, const f32x4 (&x)[D / 16], float scale, int G, int t) {
#pragma unroll
  for (int db = 0; db < D / 16; ++db) *(f32x4 *)(buf + t * (D + 4) + 16 * db + 4 * G) = x[db] * scale;
}

template <int D>
__device__ __forceinline__ void add_rows(bf16 *dst_row, const float *buf, const bf16x8 (&old)[D / 32], int G, int t) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const f32x4 a = *(const f32x4 *)(buf + t * (D + 4) + 32 * kk + 8 * G);
    const f32x4 b = *(const f32x4 *)(buf + t * (D + 4) + 32 * kk + 8 * G + 4);
    const uint2 lo = pack_bf16x4((float)old[kk][0] + a[0], (float)old[kk][1] + a[1],
                                 (float)old[kk][2] + a[2], (float)old[kk][3] + a[3]);
    const uint2 hi = pack_bf16x4((float)old[kk][4] + b[0], (float)old[kk][5] + b[1],
                                 (float)old[kk][6] + b[2], (float)old[kk][7] + b[3]);
    *(uint4 *)(dst_row + 32 * kk + 8 * G) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// Bytes of a wave's fp32 staging rows.
template <int D>
constexpr int kStageBytes = 16 * (D + 4) * 4;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Key-stationary: one wave per (batch, KV head, residue, tile of 16 key
// periods); loops over the GQA group's heads and the query-period tiles that
// have these keys as skip keys; adds the skip contributions to dk, dv.
// WITH_Q (every residue chain is one tile: P - m_min <= 16): the single query
// tile holds every query of the chain and every skip key of those queries is
// in this key tile, so the wave also adds the dq contribution and writes
// dalpha.
template <int D, bool WITH_Q>
__global__ __launch_bounds__(256) void skip_bwd_kv_kernel(Params p) {
  constexpr int LD = D + 8, NK = D / 32, ND = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 lds[4][(WITH_Q ? 3 : 2) * 16 * LD];
  static_assert(2 * 16 * LD * 2 >= kStageBytes<D>, "the fp32 staging rows fit in the q and dO slabs");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int work = blockIdx.x * 4 + wave;
  if (work >= p.nwork_kv) return;  // no block-level barrier below: waves are independent
  const int kt = work % p.nkt;
  const int r = (work / p.nkt) % p.pi;
  const int bg = work / (p.nkt * p.pi);
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int N = p.N;
  const int G = lane >> 4, t = lane & 15;
  const int k0 = 16 * kt;
  const long long ikl = (long long)r + (long long)(k0 + t) * p.pi;
  const bool kvalid = ikl < N;
  // Rows past the chain re-read row r (in range: r < pi < N) and only meet
  // masked scores; loads are unconditional so they are issued together.
  const int ik = kvalid ? (int)ikl : r;
  // a key with no query at period + m_min has no skip queries: its rows are left as the walks wrote them
  const bool kpart = kvalid && ikl + (long long)p.m_min * p.pi < N;
  const bf16 *Kp = p.k + (size_t)bg * N * D, *Vp = p.v + (size_t)bg * N * D;
  bf16 *qs = lds[wave], *os = qs + 16 * LD, *ks = os + 16 * LD;

  bf16x8 kf[NK], vf[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    kf[kk] = *(const bf16x8 *)(Kp + (size_t)ik * D + 32 * kk + 8 * G);
    vf[kk] = *(const bf16x8 *)(Vp + (size_t)ik * D + 32 * kk + 8 * G);
  }
  // the dk, dv rows the walks wrote, read now so the add at the end waits on nothing
  const size_t krow = (size_t)bg * N + ik;
  bf16x8 dk0[NK], dv0[NK];
  if (kpart) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      dk0[kk] = *(const bf16x8 *)(p.dk + krow * D + 32 * kk + 8 * G);
      dv0[kk] = *(const bf16x8 *)(p.dv + krow * D + 32 * kk + 8 * G);
    }
  }
  if (WITH_Q) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) *(bf16x8 *)(ks + t * LD + 32 * kk + 8 * G) = kf[kk];
  }
  f32x4 adk[ND], adv[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    adk[db] = f32x4{};
    adv[db] = f32x4{};
  }
  const int q_lo = k0 + p.m_min;
  const int q_hi = min(p.P - 1, k0 + 15 + p.M);
  for (int hh = 0; hh < p.grp; ++hh) {
    const size_t bh = (size_t)b * p.Hq + g * p.grp + hh;
    const bf16 *Qp = p.q + bh * N * D, *Op = p.dO + bh * N * D;
    for (int q0 = q_lo; q0 <= q_hi; q0 += 16) {
      const long long iql = (long long)r + (long long)(q0 + t) * p.pi;
      const bool qvalid = iql < N;
      const int iq = qvalid ? (int)iql : r;   // in-range row; masked below
      const size_t qrow = bh * N + iq;
      bf16x8 qa[NK], oa[NK], dqo[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        qa[kk] = *(const bf16x8 *)(Qp + (size_t)iq * D + 32 * kk + 8 * G);
        oa[kk] = *(const bf16x8 *)(Op + (size_t)iq * D + 32 * kk + 8 * G);
        if (WITH_Q) dqo[kk] = *(const bf16x8 *)(p.dq + qrow * D + 32 * kk + 8 * G);
      }
      const float c0 = -p.lse[qrow] * kLog2e;
      const float Dq = p.Dv[qrow];
      const float al = p.alpha[qrow];
      f32x4 sc = f32x4{}, dp = f32x4{};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], kf[kk], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[kk], vf[kk], dp, 0, 0, 0);
      }
      wave_lds_sync();  // the previous tile's transposed reads are done
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        *(bf16x8 *)(qs + t * LD + 32 * kk + 8 * G) = qa[kk];
        *(bf16x8 *)(os + t * LD + 32 * kk + 8 * G) = oa[kk];
      }
      // element jj: query period q0 + 4G + jj (its scalars live in lane 4G + jj), key period k0 + t
      bf16x4 pb, sb;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int src = 4 * G + jj;
        const float c0j = __shfl(c0, src, 64), Dj = __shfl(Dq, src, 64), aj = __shfl(al, src, 64);
        const int qv = __shfl((int)qvalid, src, 64);
        const int m = q0 + src - (k0 + t);
        const bool ok = kvalid && qv && m >= p.m_min && m <= p.M;
        const float pr = ok ? fast_exp2(fmaf(sc[jj], p.scale_log2, c0j)) * (1.0f - aj) : 0.f;
        pb[jj] = (bf16)pr;
        sb[jj] = (bf16)(pr * (dp[jj] - Dj));
      }
      wave_lds_sync();
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        adv[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_tr16<LD>(os, 16 * db, G, t), pb, adv[db], 0, 0, 0);
        adk[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_tr16<LD>(qs, 16 * db, G, t), sb, adk[db], 0, 0, 0);
      }
      if (WITH_Q) {
        // element jj: key period k0 + 4G + jj, query period q0 + t (this lane's query)
        f32x4 st = f32x4{}, dpt = f32x4{};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qa[kk], st, 0, 0, 0);
          dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[kk], oa[kk], dpt, 0, 0, 0);
        }
        bf16x4 dsb;
        float da = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int m = q0 + t - (k0 + 4 * G + jj);
          const bool ok = qvalid && m >= p.m_min && m <= p.M;
          const float pnp = ok ? fast_exp2(fmaf(st[jj], p.scale_log2, c0)) : 0.f;  // P / (1 - alpha)
          const float d = dpt[jj] - Dq;
          dsb[jj] = (bf16)(pnp * (1.0f - al) * d);
          da -= pnp * d;
        }
        da += wave_shfl_xor(da, 16);
        da += wave_shfl_xor(da, 32);
        f32x4 aq[ND];
#pragma unroll
        for (int db = 0; db < ND; ++db)
          aq[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_tr16<LD>(ks, 16 * db, G, t), dsb, f32x4{}, 0, 0, 0);
        // the q and dO slabs are free once the dV and dK products have read them
        float *buf = (float *)qs;
        wave_lds_sync();
        stage_rows<D>(buf, aq, p.scale, G, t);
        wave_lds_sync();
        if (qvalid) {
          add_rows<D>(p.dq + qrow * D, buf, dqo, G, t);
          if (G == 0 && p.dalpha != nullptr) p.dalpha[qrow] = da / al;
        }
      }
    }
  }
  float *buf = (float *)qs;
  wave_lds_sync();  // the last tile's transposed reads are done
  stage_rows<D>(buf, adk, p.scale, G, t);
  wave_lds_sync();
  if (kpart) add_rows<D>(p.dk + krow * D, buf, dk0, G, t);
  wave_lds_sync();
  stage_rows<D>(buf, adv, 1.0f, G, t);
  wave_lds_sync();
  if (kpart) add_rows<D>(p.dv + krow * D, buf, dv0, G, t);
}

// Query-stationary (residue chains longer than one tile): one wave per
// (batch, head, residue, tile of 16 query periods); loops over the key-period
// tiles of their skip keys; adds the dq skip contribution and writes dalpha.
template <int D>
__global__ __launch_bounds__(256) void skip_bwd_q_kernel(Params p) {
  constexpr int LD = D + 8, NK = D / 32, ND = D / 16;
  // per wave: the K rows for the transposed reads, then the fp32 staging rows
  __shared__ __attribute__((aligned(16))) float lds[4][16 * (D + 4)];
  static_assert(16 * LD * 2 <= kStageBytes<D>, "the K slab fits in the staging rows");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int work = blockIdx.x * 4 + wave;
  if (work >= p.nwork_q) return;  // no block-level barrier below
  const int tile = work % p.nqt;
  const int r = (work / p.nqt) % p.pi;
  const size_t bh = (size_t)(work / (p.nqt * p.pi));
  const int hq = (int)(bh % p.Hq), b = (int)(bh / p.Hq), g = hq / p.grp;
  const int N = p.N;
  const int G = lane >> 4, t = lane & 15;
  const int p0 = p.m_min + 16 * tile;
  const long long iql = (long long)r + (long long)(p0 + t) * p.pi;
  const bool qvalid = iql < N;
  const int iq = qvalid ? (int)iql : r;   // in-range row (r < pi < N); masked below
  const size_t qrow = bh * N + iq;
  const bf16 *Kp = p.k + (size_t)(b * p.Hkv + g) * N * D, *Vp = p.v + (size_t)(b * p.Hkv + g) * N * D;
  bf16 *ks = (bf16 *)lds[wave];
  bf16x8 qa[NK], oa[NK], dqo[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    qa[kk] = *(const bf16x8 *)(p.q + qrow * D + 32 * kk + 8 * G);
    oa[kk] = *(const bf16x8 *)(p.dO + qrow * D + 32 * kk + 8 * G);
    dqo[kk] = *(const bf16x8 *)(p.dq + qrow * D + 32 * kk + 8 * G);
  }
  const float c0 = -p.lse[qrow] * kLog2e;
  const float Dq = p.Dv[qrow];
  const float al = p.alpha[qrow];
  f32x4 aq[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) aq[db] = f32x4{};
  float da = 0.f;
  const int kt_lo = max(0, p0 - p.M), kt_hi = p0 + 15 - p.m_min;
  for (int kt = kt_lo; kt <= kt_hi; kt += 16) {
    const long long ikl = (long long)r + (long long)(kt + t) * p.pi;
    const int ik = ikl < N ? (int)ikl : r;   // rows past the chain: masked scores
    bf16x8 ka[NK], va[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      ka[kk] = *(const bf16x8 *)(Kp + (size_t)ik * D + 32 * kk + 8 * G);
      va[kk] = *(const bf16x8 *)(Vp + (size_t)ik * D + 32 * kk + 8 * G);
    }
    // element jj: key period kt + 4G + jj, query period p0 + t
    f32x4 st = f32x4{}, dpt = f32x4{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qa[kk], st, 0, 0, 0);
      dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[kk], oa[kk], dpt, 0, 0, 0);
    }
    wave_lds_sync();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) *(bf16x8 *)(ks + t * LD + 32 * kk + 8 * G) = ka[kk];
    bf16x4 dsb;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int m = p0 + t - (kt + 4 * G + jj);
      const bool ok = qvalid && m >= p.m_min && m <= p.M;
      const float pnp = ok ? fast_exp2(fmaf(st[jj], p.scale_log2, c0)) : 0.f;
      const float d = dpt[jj] - Dq;
      dsb[jj] = (bf16)(pnp * (1.0f - al) * d);
      da -= pnp * d;
    }
    wave_lds_sync();
#pragma unroll
    for (int db = 0; db < ND; ++db)
      aq[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_tr16<LD>(ks, 16 * db, G, t), dsb, aq[db], 0, 0, 0);
  }
  da += wave_shfl_xor(da, 16);
  da += wave_shfl_xor(da, 32);
  float *buf = lds[wave];
  wave_lds_sync();  // the last tile's transposed reads are done
  stage_rows<D>(buf, aq, p.scale, G, t);
  wave_lds_sync();
  if (!qvalid) return;
  add_rows<D>(p.dq + qrow * D, buf, dqo, G, t);
  if (G == 0 && p.dalpha != nullptr) p.dalpha[qrow] = da / al;
}

// Store 16 accumulator values of a 32x32 C tile (rows 8(j/4) + 4h + j%4 of the
// 32-row block db, column = this lane) as bf16, scaled, with 16-byte stores
// (half h writes elements 16jp + 8h .. +7 of each 32-block).  Both halves of
// a lane pair must be active.
template <int D>
__device__ __forceinline__ void store_rows_bf16(bf16 *dst, const f32x16 (&acc)[D / 32], float scale, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      uint2 pk[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int j4 = 2 * jp + j;
        pk[j] = pack_bf16x4(acc[db][4 * j4] * scale, acc[db][4 * j4 + 1] * scale,
                            acc[db][4 * j4 + 2] * scale, acc[db][4 * j4 + 3] * scale);
      }
      *(uint4 *)(dst + 32 * db + 16 * jp + 8 * h) = half_regroup(pk[0], pk[1]);
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
// Walk order of a block's ntiles tiles starting at tile row t_begin: for the
// window masks (every interior block has the same ntiles) the walk starts at
// the tile whose global index is 0 mod ntiles and wraps around, so blocks
// running side by side load the same tile at the same step and share it in
// L2.  Any order gives the same sums up to rounding (masks are per tile).
struct TileWalk {
  int t_begin, ntiles, rot;
  __device__ TileWalk(int tb, int nt, int mode) : t_begin(tb), ntiles(nt), rot(0) {
    if (mode == kModePi || mode == kModeWindow || mode == kModeWindowBidir) {
      const int r = (tb / BN) % nt;
      rot = r == 0 ? 0 : nt - r;
    }
  }
  __device__ __forceinline__ int row(int t) const {
    int u = t + rot;
    if (u >= ntiles) u -= ntiles;
    return t_begin + u * BN;
  }
};

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
  const TileOffsets<D> off(lane);
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
  const int t_begin = (key_lo(i0, p.mode, p.k_win, p.seg) / BN) * BN;
  const int hi_wg = key_hi(min(i0 + BM - 1, N - 1), N, p.mode, p.k_win, p.seg);
  const int ntiles = (hi_wg - t_begin) / BN + 1;
  const TileWalk walk(t_begin, ntiles, p.mode);
  // The first K/V tile goes out before the query rows: one wait covers both.
  stage_tile<D>(Kp, walk.row(0), N - 1, lds0, wave, lane);
  stage_tile<D>(Vp, walk.row(0), N - 1, lds0 + 2 * TILE, wave, lane);

  bf16x8 qf[NQF], df[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) {
    qf[kk] = qvalid ? *(const bf16x8 *)(p.q + row * D + 16 * kk + 8 * h) : bf16x8{};
    df[kk] = qvalid ? *(const bf16x8 *)(p.dO + row * D + 16 * kk + 8 * h) : bf16x8{};
  }
  float ci, Di;
  if (p.fold_prep) {
    // D_i = <dO_i, o_i>: this lane's half of the row (the chunks it holds of
    // dO), summed over the two wave halves; c_i as the prep pass forms it
    float dsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk) {
      const bf16x8 ov = qvalid ? *(const bf16x8 *)(p.o + row * D + 16 * kk + 8 * h) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf((float)df[kk][e], (float)ov[e], dsum);
    }
    Di = half_swap_sum(dsum);
    ci = 0.f;
    if (qvalid) {
      ci = -p.lse[row] * kLog2e;
      if (p.mode == kModePi && p.alpha != nullptr) ci += __log2f(p.alpha[row]);
      if (h == 0) {
        p.Dv[row] = Di;
        p.cv[row] = ci;
      }
    }
  } else {
    ci = qvalid ? p.cv[row] : 0.f;
    Di = qvalid ? p.Dv[row] : 0.f;
  }
  const int lo_i = key_lo(qi, p.mode, p.k_win, p.seg);
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const int hi_i = key_hi(qi, N, p.mode, p.k_win, p.seg);
  const bool wave_live = q0 < N;
  const int w_hi = key_hi(min(q0 + 31, N - 1), N, p.mode, p.k_win, p.seg);
  const int w_hi_first = key_hi(min(q0, N - 1), N, p.mode, p.k_win, p.seg);
  const int w_lo = key_lo(min(q0, N - 1), p.mode, p.k_win, p.seg);
  const int w_lo_last = key_lo(min(q0 + 31, N - 1), p.mode, p.k_win, p.seg);
  const bool w_allvalid = q0 + 31 < N;

  __builtin_amdgcn_s_waitcnt(0);   // query rows, row scalars and the first tile
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = walk.row(t);
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) {
      stage_tile<D>(Kp, walk.row(t + 1), N - 1, lds0 + (buf ^ 1) * TILE, wave, lane);
      stage_tile<D>(Vp, walk.row(t + 1), N - 1, lds0 + (2 + (buf ^ 1)) * TILE, wave, lane);
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
      // Masks only on tiles that some row of the wave sees in part (a
      // wave-uniform branch): a hidden key's score becomes -inf, so its
      // probability and dS are 0.
      if (!(w_allvalid && (j0 + BN - 1 <= w_hi_first) && (j0 >= w_lo_last))) {
        const int a0 = lo_i - j0 - 4 * h, span = hi_i - lo_i;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int o = 32 * kb + 8 * (jj >> 2) + (jj & 3);
            if ((unsigned)(o - a0) > (unsigned)span) s[kb][jj] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          s[kb][jj] = fast_exp2(fmaf(s[kb][jj], p.scale_log2, ci)) * (dp[kb][jj] - Di);
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
  store_rows_bf16<D>(p.dq + row * D, acc, p.scale, h);
  // rows below m_min * pi have no skip key: a zero gate gradient (the skip
  // kernels write it on the other rows)
  if (p.dalpha != nullptr && !(p.skips && qi >= p.skip_first) && h == 0) p.dalpha[row] = 0.f;
}

// Queries whose key range [key_lo(i), key_hi(i)] holds key j form the range
// [first_query(j), last_query(j)] (both ends of the key range are
// non-decreasing in i), clipped to [0, N-1].
__device__ __forceinline__ int first_query(int j, const Params &p) {
  long long f = j;
  if (p.mode == kModeWindowBidir) f = (long long)j - p.k_win;
  else if (p.mode == kModeEcpFull) f = (long long)(j / p.seg) * p.seg;
  return f > 0 ? (int)f : 0;
}

__device__ __forceinline__ int last_query(int j, const Params &p) {
  long long last;
  if (p.mode == kModeEcp || p.mode == kModeEcpFull) last = ((long long)(j / p.seg) + 2) * p.seg - 1;
  else if (p.mode == kModeSsplit) last = ((long long)(j / p.seg) + 1) * p.seg - 1;
  else last = (long long)j + p.k_win;   // pi-Attention window, window, two-sided window
  return last < p.N - 1 ? (int)last : p.N - 1;
}

// ---- dk and dv: key-stationary walk over the query tiles -------------------------
// d = 128 holds K, V (64 VGPRs) and the dK, dV accumulators (128) per lane:
// one wave per SIMD, with the 512-entry register budget that allows.
// PART 0 computes dK and dV together; at d = 128 that holds K, V and both
// accumulators (one wave per SIMD), so the launch splits into a dV pass
// (PART 1: S, P and dV^T += dO^T P; no V, no dP) and a dK pass (PART 2: S,
// dP, dS and dK^T += Q^T dS), each of which fits two waves per SIMD.
template <int D, int PART>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(Params p) {
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

  constexpr bool want_dv = PART != 2, want_dk = PART != 1;
  bf16x8 kf[NQF], vf[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) {
    kf[kk] = kvalid ? *(const bf16x8 *)(p.k + krow * D + 16 * kk + 8 * h) : bf16x8{};
    if (want_dk) vf[kk] = kvalid ? *(const bf16x8 *)(p.v + krow * D + 16 * kk + 8 * h) : bf16x8{};
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
  const int t_begin = (first_query(k0, p) / BN) * BN;
  const int ntiles = (hi_q - t_begin) / BN + 1;
  const TileWalk walk(t_begin, ntiles, p.mode);
  const int wq_hi = last_query(kw_last, p);   // last query seeing this wave's keys
  const int w_lq_first = last_query(min(j_w, N - 1), p);   // last query seeing all of them
  const int w_fq_first = first_query(min(j_w, N - 1), p);  // first query seeing any of them
  const int w_fq_last = first_query(kw_last, p);            // first query seeing all of them
  const bool w_allvalid = j_w + 31 < N;
  // Query iq sees key kj iff first_query(kj) <= iq <= last_query(kj); an
  // invalid key gets an empty range.
  const int vis_lo = kvalid ? first_query(kj, p) : -(1 << 30);
  const unsigned vis_span = kvalid ? (unsigned)(last_query(kj, p) - first_query(kj, p)) : 0u;
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
    stage_tile<D>(Qp, walk.row(0), N - 1, lds0, wave, lane);
    stage_tile<D>(Op, walk.row(0), N - 1, lds0 + 2 * TILE, wave, lane);
    stage_vec(Cp, walk.row(0), lds0 + 4 * TILE);
    stage_vec(Dp, walk.row(0), lds0 + 4 * TILE + 512);
    wait_dma();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int i0 = walk.row(t);
      const int buf = t & 1;
      const bool more = t + 1 < ntiles;
      if (more) {
        const int i1 = walk.row(t + 1);
        stage_tile<D>(Qp, i1, N - 1, lds0 + (buf ^ 1) * TILE, wave, lane);
        stage_tile<D>(Op, i1, N - 1, lds0 + (2 + (buf ^ 1)) * TILE, wave, lane);
        stage_vec(Cp, i1, lds0 + 4 * TILE + 256 * (buf ^ 1));
        stage_vec(Dp, i1, lds0 + 4 * TILE + 512 + 256 * (buf ^ 1));
      }
      // this wave's keys [j_w, kw_last] are seen by queries [w_fq_first, wq_hi]
      if (wave_live && i0 + BN - 1 >= w_fq_first && i0 <= wq_hi) {
        const char *QB = smem + buf * TILE;
        const char *OB = smem + (2 + buf) * TILE;
        const float *cq = cl + 64 * buf, *dq = cl + 128 + 64 * buf;
        // every (query, key) of the tile visible: no per-element mask
        const bool full = w_allvalid && i0 >= w_fq_last && i0 + BN - 1 <= w_lq_first;
        // The 64 queries in two halves of 32 (fewer live accumulators).
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2) {
          f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int kk = 0; kk < NQF; ++kk) {
            const bf16x8 qa = *(const bf16x8 *)(QB + 32 * qb2 * RB + off.row[kk]);
            const bf16x8 oa = *(const bf16x8 *)(OB + 32 * qb2 * RB + off.row[kk]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
            if (want_dk) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kk], dp, 0, 0, 0);
          }
          // element jj: query i0 + 32 qb2 + 8(jj/4) + 4h + jj%4, key kj
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const f32x4 cvv = *(const f32x4 *)(cq + 32 * qb2 + 8 * j4 + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * j4 + e] = fast_exp2(fmaf(s[4 * j4 + e], p.scale_log2, cvv[e]));
          }
          if (!full) {   // masks only where some query of the tile misses some key of the wave (wave-uniform branch)
            const int a0 = i0 + 32 * qb2 + 4 * h - vis_lo;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
              if ((unsigned)(a0 + 8 * (jj >> 2) + (jj & 3)) > vis_span) s[jj] = 0.f;
          }
          if (want_dk) {
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
              const f32x4 dvv = *(const f32x4 *)(dq + 32 * qb2 + 8 * j4 + 4 * h);
#pragma unroll
              for (int e = 0; e < 4; ++e) dp[4 * j4 + e] = s[4 * j4 + e] * (dp[4 * j4 + e] - dvv[e]);
            }
          }
          // dV^T += dO^T P, dK^T += Q^T dS over these 32 queries
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int kk = 2 * qb2 + k2;
            bf16x8 pb, sb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (want_dv) pb[e] = (bf16)s[8 * k2 + e];
              if (want_dk) sb[e] = (bf16)dp[8 * k2 + e];
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const char *ob = OB + 16 * kk * RB, *qbp = QB + 16 * kk * RB;
              if (want_dv) {
                const short4v olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(ob + off.tr[db][0]));
                const short4v ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(ob + off.tr[db][1]));
                adv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(olo, ohi), pb, adv[db], 0, 0, 0);
              }
              if (want_dk) {
                const short4v qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(qbp + off.tr[db][0]));
                const short4v qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(qbp + off.tr[db][1]));
                adk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(qlo, qhi), sb, adk[db], 0, 0, 0);
              }
            }
          }
        }
      }
      if (more) wait_dma();
      __syncthreads();
    }
  }
  if (!kvalid) return;
  if (want_dk) store_rows_bf16<D>(p.dk + krow * D, adk, p.scale, h);
  if (want_dv) store_rows_bf16<D>(p.dv + krow * D, adv, 1.0f, h);
}

template <int D>
hipError_t launch_t(const BwdArgs &a, hipStream_t s) {
  Params p;
  p.q = (const bf16 *)a.q; p.k = (const bf16 *)a.k; p.v = (const bf16 *)a.v; p.o = (const bf16 *)a.o;
  p.dO = (const bf16 *)a.dO; p.alpha = a.alpha; p.lse = a.lse;
  p.dq = (bf16 *)a.dq; p.dk = (bf16 *)a.dk; p.dv = (bf16 *)a.dv; p.dalpha = a.dalpha;
  p.Dv = a.Dv; p.cv = a.cv;
  p.skips = a.skips;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N; p.mode = a.mode; p.k_win = a.k_win; p.pi = a.pi;
  p.M = a.M; p.m_min = a.m_min; p.seg = a.seg; p.grp = a.Hq / a.Hkv;
  p.nqb = (a.N + BM - 1) / BM;
  p.nkb = (a.N + BM - 1) / BM;
  p.scale = a.score_scale > 0.f ? a.score_scale : 1.0f / sqrtf((float)D);
  p.scale_log2 = kLog2e * p.scale;
  p.out_gate = (const bf16 *)a.out_gate;
  p.dgate = (bf16 *)a.dgate;
  p.dO_gated = (bf16 *)a.dO_gated;
  const long long rows = (long long)a.B * a.Hq * a.N;
  p.P = (a.N + a.pi - 1) / (a.pi > 0 ? a.pi : 1);
  p.skip_first = 0;
  p.nqt = p.nkt = p.nwork_q = p.nwork_kv = 0;
  if (p.skips) {
    // skips exist, so m_min * pi < N
    p.skip_first = a.m_min * a.pi;
    p.nqt = p.nkt = (p.P - a.m_min + 15) / 16;
    const long long wq = (long long)a.B * a.Hq * a.pi * p.nqt;
    if (wq > (1LL << 30)) return hipErrorInvalidValue;   // wave count beyond the 1-D grid (before any launch)
    p.nwork_q = (int)wq;
    p.nwork_kv = (int)((long long)a.B * a.Hkv * a.pi * p.nkt);
  }
  p.fold_prep = p.out_gate == nullptr;
  if (!p.fold_prep)
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0, s, p, rows);
  if (p.out_gate != nullptr) p.dO = p.dO_gated;   // the rest differentiate the ungated attention
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(a.B * a.Hq * p.nqb), dim3(256), 0, s, p);
  // d = 64: one pass (two waves per SIMD; split passes measured 20 % slower
  // there).  d = 128: the dV and dK passes (two waves each, against one for
  // the joint kernel).
  if constexpr (D == 64) {
    hipLaunchKernelGGL((bwd_dkv_kernel<D, 0>), dim3(a.B * a.Hkv * p.nkb), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((bwd_dkv_kernel<D, 1>), dim3(a.B * a.Hkv * p.nkb), dim3(256), 0, s, p);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, 2>), dim3(a.B * a.Hkv * p.nkb), dim3(256), 0, s, p);
  }
  // The skip-key contributions last: they read D_i (formed above) and add
  // into the gradients the walks have written.
  if (p.skips) {
    if (p.nqt == 1) {
      hipLaunchKernelGGL((skip_bwd_kv_kernel<D, true>), dim3((p.nwork_kv + 3) / 4), dim3(256), 0, s, p);
    } else {
      hipLaunchKernelGGL((skip_bwd_kv_kernel<D, false>), dim3((p.nwork_kv + 3) / 4), dim3(256), 0, s, p);
      hipLaunchKernelGGL((skip_bwd_q_kernel<D>), dim3((p.nwork_q + 3) / 4), dim3(256), 0, s, p);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  return a.d == 64 ? launch_t<64>(a, s) : launch_t<128>(a, s);
}

}  // namespace sa
