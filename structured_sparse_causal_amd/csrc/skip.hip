// skip.hip -- periodic skip keys of pi-Attention as a residue-class pass (gfx950).
//
// pi-Attention (section 2, item 2) lets query i attend i - m*pi for m = 1..M;
// the keys that lie below the causal window [i-k, i] are those with
// m*pi > k, i.e. m >= m_min = floor(k/pi) + 1.  Query i and its skip keys share
// the residue r = i mod pi: within one residue class, queries at periods
// p = (i - r)/pi attend the earlier periods p - m.  For a fixed residue this is
// a small dense band problem, so a wave gathers (strided gather, section 2
// item 2) 16 query periods and 16 key periods of one residue and runs it on
// the matrix cores: S^T = K Q^T with v_mfma_f32_16x16x32_bf16, band mask
// m in [m_min, M], log-prior log(1 - alpha_i) (item 3), then O^T = V^T P^T with
// v_mfma_f32_16x16x16bf16_1k.  The pass writes, per query with at least one
// skip key, the partial softmax state (running max in log2 units, sum,
// unnormalised accumulator); the prefill kernel starts from it, so the union
// of local and skip keys gets a single softmax.
//
// The fp32 I/O variant (small, correctness-first inputs) uses a plain per-query
// loop on the vector ALUs.
#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

struct Params {
  const void *q, *k, *v;
  const float *alpha;
  float *ml;
  void *acc;
  int N, Hq, Hkv, pi, M, m_min;
  int P;          // periods per residue: ceil(N / pi)
  int ntiles;     // query-period tiles of 16 per residue
  int nwork;      // B*Hq*pi*ntiles work items (one per wave)
  float scale_log2;
  FusedOpts opt;  // cosine (keys arrive normalised) and the query-driven gate
};

// log2(1 - sigmoid(z)) = log2(sigmoid(-z)) without overflow for large |z|.
__device__ __forceinline__ float log2_one_minus_sigmoid(float z) {
  return z <= 0.f ? -__log2f(1.0f + fast_exp2(z * kLog2e)) : -z * kLog2e - __log2f(1.0f + fast_exp2(-z * kLog2e));
}

// Loads of one key tile of a residue chain: the K operand row kt + t of this
// lane and its share of the 16 V rows.  Unconditional: rows past the chain
// re-read row `safe` (in range); they only ever meet masked scores.  (A
// predicated load makes the compiler wait for it right after issuing it.)
template <int D>
struct KeyTile {
  bf16x8 k[D / 32];
  u32x4 v[D / 32];
};

template <int D>
__device__ __forceinline__ void load_key_tile(KeyTile<D> &kt_regs, const bf16 *Kp, const bf16 *Vp, int kt, int r,
                                              int safe, const Params &p, int lane, int G, int t) {
  const int pk = kt + t;
  const long long ik = (long long)r + (long long)pk * p.pi;
  const int ik_ld = (pk < p.P && ik < p.N) ? (int)ik : safe;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) kt_regs.k[kk] = *(const bf16x8 *)(Kp + (size_t)ik_ld * D + 32 * kk + 8 * G);
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    const int ci = lane + 64 * u, row = ci / (D / 8), col = (ci % (D / 8)) * 8;
    const int pr = kt + row;
    const long long ir = (long long)r + (long long)pr * p.pi;
    const int ir_ld = (pr < p.P && ir < p.N) ? (int)ir : safe;
    kt_regs.v[u] = *(const u32x4 *)(Vp + (size_t)ir_ld * D + col);
  }
}

// Eight waves (eight consecutive residues) per workgroup: each period's rows of
// the group are one 1 KB run (d = 64), fetched together (-1 % against four).
constexpr int kSkipWaves = 8;

template <int D>
__global__ __launch_bounds__(64 * kSkipWaves) void skip_bf16_kernel(Params p) {
  constexpr int LD = D + 8;
  __shared__ __attribute__((aligned(16))) bf16 Vs[kSkipWaves][16 * LD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int work = blockIdx.x * kSkipWaves + wave;
  if (work >= p.nwork) return;  // no block-level barrier below: waves are independent
  const int tile = work % p.ntiles;
  const int r = (work / p.ntiles) % p.pi;
  const int bh = work / (p.ntiles * p.pi);
  const int hq = bh % p.Hq, b = bh / p.Hq, g = hq / (p.Hq / p.Hkv);
  const int N = p.N;
  const int G = lane >> 4, t = lane & 15;
  const int p0 = p.m_min + 16 * tile;         // first query period of this tile
  const int pq = p0 + t;                       // query period of lane column t
  const int iq = r + pq * p.pi;                // its position
  const bool qvalid = pq < p.P && iq < N;

  const bf16 *Qp = (const bf16 *)p.q + (size_t)bh * N * D;
  const bf16 *Kp = (const bf16 *)p.k + (size_t)(b * p.Hkv + g) * N * D;
  const bf16 *Vp = (const bf16 *)p.v + (size_t)(b * p.Hkv + g) * N * D;

  // Issue the query row, its gate input and the first key tile together; the
  // prologue below waits for them once.  Row r is in range (r < pi, and some
  // position has a skip key, so pi < N).
  // (Key tile first: any wait the compiler places for the query covers it too.)
  const int kt_lo = max(0, p0 - p.M);
  const int kt_hi = p0 + 15 - p.m_min;
  KeyTile<D> tl;
  load_key_tile<D>(tl, Kp, Vp, kt_lo, r, r, p, lane, G, t);
  const int iq_ld = qvalid ? iq : r;
  bf16x8 qf[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) qf[kk] = *(const bf16x8 *)(Qp + (size_t)iq_ld * D + 32 * kk + 8 * G);
  const float a_in = p.opt.gate_w == nullptr ? p.alpha[(size_t)bh * N + iq_ld] : 0.5f;
  float bias = -INFINITY;  // log2(1 - alpha)
  if (qvalid && p.opt.gate_w == nullptr) bias = __log2f(1.0f - a_in);
  float sl2 = p.scale_log2;
  // this lane holds dims 32kk + 8G .. +7 of query column t; the four lane
  // groups G together hold the row
  if (p.opt.cosine) {
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)qf[kk][e], (float)qf[kk][e], ss);
    ss += wave_shfl_xor(ss, 16);
    ss += wave_shfl_xor(ss, 32);
    sl2 *= rsqrtf(ss);
  }
  if (p.opt.gate_w != nullptr) {   // alpha = sigmoid(<w_h, q_i> + b_h)
    const int hg = (p.opt.gate_bh0 + bh) % p.opt.gate_hq;
    const float *w = p.opt.gate_w + (size_t)hg * D + 8 * G;
    f32x4 wv[D / 32][2];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      wv[kk][0] = *(const f32x4 *)(w + 32 * kk);
      wv[kk][1] = *(const f32x4 *)(w + 32 * kk + 4);
    }
    float z = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) z = fmaf((float)qf[kk][e], wv[kk][e >> 2][e & 3], z);
    z += wave_shfl_xor(z, 16);
    z += wave_shfl_xor(z, 32);
    if (qvalid) bias = log2_one_minus_sigmoid(z + p.opt.gate_b[hg]);
  }

  f32x4 acc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc[db] = f32x4{};
  float m_run = kNegBig, l_run = 0.f;
  bf16 *vs = Vs[wave];

  for (int kt = kt_lo; kt <= kt_hi; kt += 16) {
    if (kt != kt_lo) load_key_tile<D>(tl, Kp, Vp, kt, r, r, p, lane, G, t);
    // Key periods kt + 4G + jj (score rows), kt + t (operand rows).
    f32x4 s = f32x4{};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl.k[kk], qf[kk], s, 0, 0, 0);
    // Stage the 16 value rows of this key tile in this wave's LDS slab.
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const int ci = lane + 64 * u, row = ci / (D / 8), col = (ci % (D / 8)) * 8;
      *(u32x4 *)(vs + row * LD + col) = tl.v[u];
    }
    // Band mask: key period pk' = kt + 4G + jj is a skip key of query period pq
    // iff m = pq - pk' lies in [m_min, M].
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int m = pq - (kt + 4 * G + jj);
      const bool ok = qvalid && m >= p.m_min && m <= p.M;
      s[jj] = ok ? s[jj] * sl2 + bias : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float mr = fmaxf(m_run, mx);
    const float f = fast_exp2(m_run - mr);
    l_run *= f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc[db] *= f;
    m_run = mr;
    bf16x4 pb;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float pv = fast_exp2(s[jj] - m_run);
      l_run += pv;
      pb[jj] = (bf16)pv;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T over the 16 key periods (K = 16).
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const bf16 *src = vs + (4 * G + (t >> 2)) * LD + 16 * db + 4 * (t & 3);
      const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)src);
      const bf16x4 a = as_bf16x4(x);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  l_run += wave_shfl_xor(l_run, 16);
  l_run += wave_shfl_xor(l_run, 32);
  if (!qvalid) return;
  const size_t row = (size_t)bh * N + iq;
  if (G == 0) *(float2 *)(p.ml + 2 * row) = make_float2(m_run, l_run);
  // Accumulators are stored in bf16 (the I/O precision): half the workspace
  // traffic; the relative rounding (2^-9) applies to the skip share only.
  bf16 *ap = (bf16 *)p.acc + row * D;
  // 16-byte stores: the two 16-blocks of each 32-span regrouped between lane rows
#pragma unroll
  for (int dp = 0; dp < D / 32; ++dp)
    *(uint4 *)(ap + 32 * dp + 8 * (G >> 1) + 16 * (G & 1)) =
        row_regroup(pack_bf16x4(acc[2 * dp][0], acc[2 * dp][1], acc[2 * dp][2], acc[2 * dp][3]),
                    pack_bf16x4(acc[2 * dp + 1][0], acc[2 * dp + 1][1], acc[2 * dp + 1][2], acc[2 * dp + 1][3]));
}

// fp32 I/O: one thread per query row, plain loops.
template <int D>
__global__ __launch_bounds__(128) void skip_f32_kernel(Params p, int first, long long rows) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows) return;
  const int per_head = p.N - first;
  const int bh = (int)(idx / per_head);
  const int i = first + (int)(idx % per_head);
  const int hq = bh % p.Hq, b = bh / p.Hq, g = hq / (p.Hq / p.Hkv);
  const float *Qp = (const float *)p.q + ((size_t)bh * p.N + i) * D;
  const float *Kp = (const float *)p.k + (size_t)(b * p.Hkv + g) * p.N * D;
  const float *Vp = (const float *)p.v + (size_t)(b * p.Hkv + g) * p.N * D;
  float bias, sl2 = p.scale_log2;
  if (p.opt.gate_w != nullptr) {   // alpha = sigmoid(<w_h, q_i> + b_h)
    const int hg = (p.opt.gate_bh0 + bh) % p.opt.gate_hq;
    float z = p.opt.gate_b[hg];
    for (int c = 0; c < D; ++c) z = fmaf(Qp[c], p.opt.gate_w[(size_t)hg * D + c], z);
    bias = log2_one_minus_sigmoid(z);
  } else {
    bias = __log2f(1.0f - p.alpha[(size_t)bh * p.N + i]);
  }
  if (p.opt.cosine) {   // keys arrive normalised; 1/|q_i| joins the scale
    float ss = 0.f;
    for (int c = 0; c < D; ++c) ss = fmaf(Qp[c], Qp[c], ss);
    sl2 *= rsqrtf(ss);
  }
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  for (int m = p.m_min; m <= p.M; ++m) {
    const int j = i - m * p.pi;
    if (j < 0) break;
    float dot = 0.f;
    for (int c = 0; c < D; ++c) dot = fmaf(Qp[c], Kp[(size_t)j * D + c], dot);
    const float sc = dot * sl2 + bias;
    const float mr = fmaxf(m_run, sc);
    const float f = fast_exp2(m_run - mr);
    const float pv = fast_exp2(sc - mr);
    l_run = l_run * f + pv;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = acc[c] * f + pv * Vp[(size_t)j * D + c];
    m_run = mr;
  }
  const size_t row = (size_t)bh * p.N + i;
  p.ml[2 * row] = m_run;
  p.ml[2 * row + 1] = l_run;
#pragma unroll
  for (int c = 0; c < D; ++c) ((float *)p.acc)[row * D + c] = acc[c];
}

template <int D>
hipError_t launch_t(const SkipArgs &a, hipStream_t s) {
  Params p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.alpha = a.alpha; p.ml = a.ml; p.acc = a.acc;
  p.N = a.N; p.Hq = a.Hq; p.Hkv = a.Hkv; p.pi = a.pi; p.M = a.M; p.m_min = a.m_min;
  p.P = (a.N + a.pi - 1) / a.pi;
  p.opt = a.opt;
  p.scale_log2 = kLog2e * (a.opt.score_scale > 0.f ? a.opt.score_scale : 1.0f / sqrtf((float)D));
  const int first = a.m_min * a.pi;  // first position with a skip key
  if (first >= a.N) return hipSuccess;
  if (a.dtype == kBF16) {
    p.ntiles = (p.P - a.m_min + 15) / 16;
    const long long nwork = (long long)a.B * a.Hq * a.pi * p.ntiles;
    p.nwork = (int)nwork;
    hipLaunchKernelGGL((skip_bf16_kernel<D>), dim3((p.nwork + kSkipWaves - 1) / kSkipWaves), dim3(64 * kSkipWaves), 0, s, p);
  } else {
    p.ntiles = 0;
    p.nwork = 0;
    const long long rows = (long long)a.B * a.Hq * (a.N - first);
    hipLaunchKernelGGL((skip_f32_kernel<D>), dim3((unsigned)((rows + 127) / 128)), dim3(128), 0, s, p,
                       first, rows);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skip(const SkipArgs &a, hipStream_t s) {
  return a.d == 64 ? launch_t<64>(a, s) : launch_t<128>(a, s);
}

}  // namespace sa
