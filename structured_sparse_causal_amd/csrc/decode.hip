// decode.hip -- single-token decode over a KV cache for gfx950 (memory bound).
//
// Each sequence b has ONE new query per query head at position i = len_b - 1,
// attending the key set of i (pi-Attention window + periodic skips, the
// window alone, or the ECP pair of half-segments).  Grouped-query attention
// (attention branch of the hybrid GSS-Transformer page, methodology item 1):
// the query heads of one KV head share every key/value row, so one workgroup
// serves a (sequence, KV head, head chunk of <= 16, key split) and reads each
// attended cache row once.  The window range is cut into `n_wsplit` splits of
// `chunk` rows; the skip keys (strided rows i - m*pi) form one extra split.
// A split writes its partial softmax state (max in log2 units, sum,
// unnormalised accumulator) per query head; a combine kernel merges the splits
// exactly (log-sum-exp merge) and normalises.
//
// Per wave and 16 rows: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows are the
// A operand, loaded straight from HBM in operand layout; queries of the group
// are the columns), online softmax per head column, then O^T += V^T P^T on
// v_mfma_f32_16x16x16bf16_1k with the V^T fragment read transposed from a
// per-wave LDS slab (ds_read_b64_tr_b16).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace sa {
namespace {

constexpr float kTau = 8.0f;

struct Params {
  const void *q, *kc, *vc;
  const int *lens;
  const float *alpha;
  void *o;
  float *ws;
  int Hq, Hkv, Lmax, mode, k_win, pi, M, seg, m_min;
  int n_wsplit, chunk, nsplit, hchunks, grp;
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

// Rows of this split: count and position of row r.
struct SplitRows {
  int count, base, stride;  // position(r) = base - r*stride for skips, base + r otherwise
  bool skip;
  __device__ __forceinline__ int pos(int r) const { return skip ? base - r * stride : base + r; }
};

__device__ __forceinline__ SplitRows split_rows(const Params &p, int i, int split) {
  SplitRows sr;
  const int lo = key_lo(i, p.mode, p.k_win, p.seg);
  if (split < p.n_wsplit) {
    const int a = lo + split * p.chunk;
    const int e = min(a + p.chunk, i + 1);
    sr.count = e > a ? e - a : 0;
    sr.base = a;
    sr.stride = 0;
    sr.skip = false;
  } else {
    // Skip keys i - m*pi, m = m_min..M, that are >= 0 (all lie below lo).
    const int first = i - p.m_min * p.pi;
    int cnt = 0;
    if (p.mode == kModePi && p.M >= p.m_min && first >= 0) cnt = min(p.M - p.m_min, first / p.pi) + 1;
    sr.count = cnt;
    sr.base = first;
    sr.stride = p.pi;
    sr.skip = true;
  }
  return sr;
}

constexpr int kWaves = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(Params p) {
  constexpr bool kBF = sizeof(T) == 2;
  constexpr int LD = D + 8;
  constexpr int NDB = D / 16;
  __shared__ __attribute__((aligned(16))) T Vs[kWaves][kBF ? 16 * LD : 1];
  __shared__ float red_m[kWaves][16], red_l[kWaves][16];
  __shared__ float red_acc[kWaves][16][D + 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = lane >> 4, t = lane & 15;
  const int split = blockIdx.x;
  const int g = blockIdx.y / p.hchunks, hc = blockIdx.y % p.hchunks;
  const int b = blockIdx.z;
  const int len = p.lens[b];
  const bool len_ok = len >= 1 && len <= p.Lmax;
  const int i = len_ok ? len - 1 : 0;
  const int head = 16 * hc + t;               // index inside the GQA group
  const bool hvalid = head < p.grp;
  const int hq = g * p.grp + head;
  const size_t kvoff = (size_t)(b * p.Hkv + g) * p.Lmax * D;
  const T *Kp = (const T *)p.kc + kvoff;
  const T *Vp = (const T *)p.vc + kvoff;
  const T *Qp = (const T *)p.q + ((size_t)b * p.Hq + hq) * D;

  SplitRows sr = split_rows(p, i, split);
  if (!len_ok) sr.count = 0;

  float bias = 0.f;
  if (p.mode == kModePi && p.alpha != nullptr && hvalid) {
    const float a = p.alpha[(size_t)b * p.Hq + hq];
    bias = sr.skip ? __log2f(1.0f - a) : __log2f(a);
  }

  // Query fragment (B operand): column t = query head of the group.
  constexpr int NQF = kBF ? D / 32 : D / 4;
  typedef typename std::conditional<kBF, bf16x8, float>::type QFrag;
  QFrag qf[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) {
    if constexpr (kBF) qf[kk] = hvalid ? *(const bf16x8 *)(Qp + 32 * kk + 8 * G) : bf16x8{};
    else qf[kk] = hvalid ? (float)Qp[4 * kk + G] : 0.f;
  }

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
  float m_run = kNegBig, l_run = 0.f;
  T *vs = Vs[wave];

  for (int r0 = 16 * wave; r0 < sr.count; r0 += 16 * kWaves) {
    // ---- scores for rows r0 + 4G + jj (C layout), operand row r0 + t ---------
    const bool rvalid = r0 + t < sr.count;
    const int prow = sr.pos(min(r0 + t, sr.count - 1));
    f32x4 s = f32x4{};
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk) {
      if constexpr (kBF) {
        const bf16x8 a = rvalid ? *(const bf16x8 *)(Kp + (size_t)prow * D + 32 * kk + 8 * G) : bf16x8{};
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], s, 0, 0, 0);
      } else {
        const float a = rvalid ? (float)Kp[(size_t)prow * D + 4 * kk + G] : 0.f;
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[kk], s, 0, 0, 0);
      }
    }
    if constexpr (kBF) {
      // Stage the 16 value rows for the transposed read.
#pragma unroll
      for (int ci = lane; ci < 16 * D / 8; ci += 64) {
        const int row = ci / (D / 8), col = (ci % (D / 8)) * 8;
        uint4 vv = make_uint4(0, 0, 0, 0);
        if (r0 + row < sr.count) vv = *(const uint4 *)(Vp + (size_t)sr.pos(r0 + row) * D + col);
        *(uint4 *)(vs + row * LD + col) = vv;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      s[jj] = (r0 + 4 * G + jj < sr.count) ? s[jj] : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = mx * p.scale_log2 + bias;
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
    for (int jj = 0; jj < 4; ++jj) {
      s[jj] = fast_exp2(fmaf(s[jj], p.scale_log2, nb));
      l_run += s[jj];
    }
    if constexpr (kBF) {
      bf16x4 pb;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pb[jj] = (bf16)s[jj];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const T *src = vs + (4 * G + (t >> 2)) * LD + 16 * db + 4 * (t & 3);
        const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)src);
        const bf16x4 a = as_bf16x4(x);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, acc[db], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      // k index of the 16x16x4 f32 product = lane group G <-> row r0 + 4G + jj.
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rr = r0 + 4 * G + jj;
        const bool ok = rr < sr.count;
        const size_t vrow = (size_t)sr.pos(ok ? rr : 0) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const float a = ok ? (float)Vp[vrow + 16 * db + t] : 0.f;
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s[jj], acc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- merge the four waves, then write this split's partial state -------
  l_run += wave_shfl_xor(l_run, 16);
  l_run += wave_shfl_xor(l_run, 32);
  if (G == 0) {
    red_m[wave][t] = m_run;
    red_l[wave][t] = l_run;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) red_acc[wave][t][16 * db + 4 * G + jj] = acc[db][jj];
  __syncthreads();
  // Thread (head hh, dims) merges: 256 threads = 16 heads x 16 dim lanes.
  const int hh = threadIdx.x >> 4, dl = threadIdx.x & 15;
  if (16 * hc + hh >= p.grp) return;
  float mw[kWaves], mstar = kNegBig;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = red_m[w][hh];
    mstar = fmaxf(mstar, mw[w]);
  }
  float fw[kWaves], lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    fw[w] = fast_exp2(mw[w] - mstar);
    lsum += red_l[w][hh] * fw[w];
  }
  const int hq_out = g * p.grp + 16 * hc + hh;
  float *wp = p.ws + (((size_t)b * p.Hq + hq_out) * p.nsplit + split) * (D + 2);
  if (!len_ok) mstar = NAN;
  if (dl == 0) {
    wp[0] = mstar;
    wp[1] = lsum;
  }
  for (int dim = dl; dim < D; dim += 16) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) a += red_acc[w][hh][dim] * fw[w];
    wp[2 + dim] = a;
  }
}

// Merge the split partials of one (sequence, query head) and normalise.
template <typename T, int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(Params p) {
  const int row = blockIdx.x;  // b*Hq + hq
  const float *wp = p.ws + (size_t)row * p.nsplit * (D + 2);
  float mstar = kNegBig;
  for (int s = 0; s < p.nsplit; ++s) mstar = fmaxf(mstar, wp[s * (D + 2)]);
  bool bad = false;
  for (int s = 0; s < p.nsplit; ++s) bad |= (wp[s * (D + 2)] != wp[s * (D + 2)]);
  float l = 0.f;
  for (int s = 0; s < p.nsplit; ++s) l += wp[s * (D + 2) + 1] * fast_exp2(wp[s * (D + 2)] - mstar);
  for (int dim = threadIdx.x; dim < D; dim += blockDim.x) {
    float a = 0.f;
    for (int s = 0; s < p.nsplit; ++s) a += wp[s * (D + 2) + 2 + dim] * fast_exp2(wp[s * (D + 2)] - mstar);
    const float o = bad ? NAN : a / l;
    T *op = (T *)p.o + (size_t)row * D + dim;
    if constexpr (sizeof(T) == 2) *(unsigned short *)op = f32_to_bf16_bits(o);
    else *op = o;
  }
}

template <typename T, int D>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
  Params p;
  p.q = a.q; p.kc = a.kc; p.vc = a.vc; p.lens = a.lens; p.alpha = a.alpha; p.o = a.o; p.ws = a.ws;
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.Lmax = a.Lmax; p.mode = a.mode; p.k_win = a.k_win; p.pi = a.pi;
  p.M = a.M; p.seg = a.seg; p.m_min = a.m_min;
  p.n_wsplit = a.n_wsplit; p.chunk = a.chunk; p.nsplit = a.nsplit;
  p.grp = a.Hq / a.Hkv;
  p.hchunks = (p.grp + 15) / 16;
  p.scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(p.nsplit, a.Hkv * p.hchunks, a.B), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.B * a.Hq), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.dtype == kBF16) return a.d == 64 ? launch_t<bf16, 64>(a, s) : launch_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_t<float, 64>(a, s) : launch_t<float, 128>(a, s);
}

}  // namespace sa
