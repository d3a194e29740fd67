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
// bf16: each wave streams 16-row groups (K and V in whole cache lines, with
// non-temporal loads, one group in flight while the previous one is consumed),
// stages them in a per-wave LDS slab, computes S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16 (query heads of the group as columns), runs the
// online softmax per head, and accumulates O with v_mfma_f32_4x4x4bf16_1k
// (4 query heads x 64 dims per instruction).  fp32 uses the 16x16x4 f32
// product with operands read from memory.  The four waves' partial states are
// merged pairwise through LDS at the end.
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
  int R, page_shift, num_pages, max_pages;   // ring / paged cache layouts
  const int *table;
  FusedOpts opt;    // bf16: score scale, cosine, query-driven gate, output gate
  int walk_splits;  // bf16: one workgroup walks every split and writes o (no combine)
};

__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e)); }


// Rows of this split: count and position of row r.
struct SplitRows {
  int count, base, step;  // window splits: position(r) = base + r (local keys)
  int qrow;               // last split: row 0 is the query row qrow (local),
  bool last;              // rows r >= 1 are skips at base + r*step, step = -pi
  __device__ __forceinline__ int pos(int r) const { return (last && r == 0) ? qrow : base + r * step; }
  __device__ __forceinline__ bool skip_row(int r) const { return last && r != 0; }
};

// Rows of split `split` for the query at position i.  The window rows below i
// are cut into n_wsplit splits of `chunk` rows; the last split holds the query
// row itself and the skip keys i - m*pi (m = m_min..M, >= 0, all below the
// window), so no split is nearly empty.
__device__ __forceinline__ SplitRows split_rows(const Params &p, int i, int split) {
  SplitRows sr;
  const int lo = key_lo(i, p.mode, p.k_win, p.seg);
  sr.qrow = i;
  if (split < p.n_wsplit) {
    const int a = lo + split * p.chunk;
    const int e = min(a + p.chunk, i);
    sr.count = e > a ? e - a : 0;
    sr.base = a;
    sr.step = 1;
    sr.last = false;
  } else {
    const int first = i - p.m_min * p.pi;
    int cnt = 0;
    if (p.mode == kModePi && p.M >= p.m_min && first >= 0) cnt = min(p.M - p.m_min, first / p.pi) + 1;
    sr.count = 1 + cnt;
    sr.base = first + p.pi;
    sr.step = -p.pi;
    sr.last = true;
  }
  return sr;
}

// All window rows below i as one split (the union of the window splits, in the
// same order).  The window splits are multiples of 64 rows, so a wave taking
// every fourth 16-row group meets the same rows in the same order either way.
__device__ __forceinline__ SplitRows window_rows(const Params &p, int i) {
  SplitRows sr;
  const int lo = key_lo(i, p.mode, p.k_win, p.seg);
  sr.qrow = i;
  sr.count = i > lo ? i - lo : 0;
  sr.base = lo;
  sr.step = 1;
  sr.last = false;
  return sr;
}

// Physical row (relative to the per-layout base pointer) of row r of a split.
//   contiguous [B,Hkv,Lmax,d]: base = (b,g) slice, row = position;
//   ring [B,Hkv,R,d]: base = (b,g) slice, row = position mod R (a split's rows
//     are base + r*step with |r*step| < R, so one wrap of the slot of `base`);
//   paged [num_pages,Hkv,P,d]: base = pool, row = (page*Hkv + g)*P + position % P,
//     the page read by lane shuffle from the split's block-table entries that
//     each wave loads up front (lane l: page l of a window split, or the page of
//     row l of the query/skip split).
template <int LAYOUT>
struct RowMap {
  SplitRows sr;
  int sbase, qslot, R;             // ring
  int ptab, page0, g, Hkv, P, sh;  // paged
  __device__ __forceinline__ int phys(int r) const {
    if constexpr (LAYOUT == kCacheContig) {
      return sr.pos(r);
    } else if constexpr (LAYOUT == kCacheRing) {
      int x = sbase + r * sr.step;
      x = x < 0 ? x + R : x;
      x = x >= R ? x - R : x;
      return (sr.last && r == 0) ? qslot : x;
    } else {
      const int pos = sr.pos(r);
      const int idx = sr.last ? r : (pos >> sh) - page0;
      const int page = __shfl(ptab, idx, 64);
      return (page * Hkv + g) * P + (pos & (P - 1));
    }
  }
};

__device__ __forceinline__ int mod_pos(long long x, int R) {
  const long long m = x % R;
  return (int)(m < 0 ? m + R : m);
}

// Builds the row map of a split; `bad` is set (uniformly across the
// workgroup) when a block-table entry the split needs is out of range.
template <int LAYOUT>
__device__ __forceinline__ RowMap<LAYOUT> make_rowmap(const Params &p, const SplitRows &sr, int b, int g, int lane,
                                                      bool &bad) {
  RowMap<LAYOUT> rm;
  rm.sr = sr;
  bad = false;
  if constexpr (LAYOUT == kCacheRing) {
    rm.R = p.R;
    rm.sbase = mod_pos(sr.base, p.R);
    rm.qslot = mod_pos(sr.qrow, p.R);
  } else if constexpr (LAYOUT == kCachePaged) {
    rm.g = g;
    rm.Hkv = p.Hkv;
    rm.sh = p.page_shift;
    rm.P = 1 << p.page_shift;
    rm.page0 = sr.base >> p.page_shift;
    rm.ptab = 0;
    if (sr.count > 0) {
      int pg;
      bool need;
      if (!sr.last) {
        pg = rm.page0 + lane;
        need = pg <= ((sr.base + sr.count - 1) >> p.page_shift);
      } else {
        need = lane < sr.count;
        pg = sr.pos(need ? lane : 0) >> p.page_shift;
      }
      const int e = need ? p.table[(size_t)b * p.max_pages + pg] : 0;
      rm.ptab = e;
      bad = __any(need && (e < 0 || e >= p.num_pages));
    }
  }
  return rm;
}

constexpr int kWaves = 4;
constexpr int kRing = 2;   // 16-row groups per wave held in registers (kRing - 1 in flight)

// One 16-row group of a wave in flight: the 16 rows of K and of V as 16-byte
// chunks (chunk lane + 64*u of the row-major 16 x D block, so every load
// instruction reads whole 128-byte lines).  Cache rows are read exactly once,
// with non-temporal loads: on this access pattern (a 0.5 MB run per
// (sequence, KV head) at an 8 MB stride) they stream at about 7 TB/s against
// about 5.8 TB/s for cached loads.
template <int D>
struct Group {
  static constexpr int NC = D / 32;   // chunks per lane per tensor
  u32x4 k[NC], v[NC];
};

// Loads are unconditional (no per-lane branches, which would make the
// compiler wait on each load right after issuing it): rows past the split's
// end re-read its last row (scores masked, probabilities 0) and an empty split
// reads `fallback`, an in-range row.
template <int D, int LAYOUT>
__device__ __forceinline__ Group<D> load_group(const bf16 *Kp, const bf16 *Vp, const RowMap<LAYOUT> &rm, int r0,
                                               int lane, int fallback) {
  Group<D> g;
  const int last = rm.sr.count - 1;
#pragma unroll
  for (int u = 0; u < Group<D>::NC; ++u) {
    const int ci = lane + 64 * u, row = ci / (D / 8), col = (ci % (D / 8)) * 8;
    const size_t off = (size_t)(last >= 0 ? rm.phys(min(r0 + row, last)) : fallback) * D + col;
    g.k[u] = load_once16(Kp + off);
    g.v[u] = load_once16(Vp + off);
  }
  return g;
}

// Workspace entry of one (sequence, query head, split): max (log2 units), sum,
// two pad words, then the d-wide unnormalised accumulator (16-byte aligned).
template <int D>
constexpr int ws_stride() { return D + 4; }

// fp32 I/O: per wave and 16 rows, S^T = K Q^T on v_mfma_f32_16x16x4f32 and
// O^T += V^T P^T on the same instruction, operands read straight from memory;
// the four waves' partial states are merged pairwise through LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(Params p) {
  constexpr int NDB = D / 16;
  constexpr int kSlotBytes = 64 * NDB * 16 + 2 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[2 * kSlotBytes];

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
  const float *Kp = (const float *)p.kc + kvoff;
  const float *Vp = (const float *)p.vc + kvoff;
  const float *Qp = (const float *)p.q + ((size_t)b * p.Hq + hq) * D;

  SplitRows sr = split_rows(p, i, split);
  if (!len_ok) sr.count = 0;

  float bias_loc = 0.f, bias_skip = 0.f;   // log2 priors of local and skip keys
  if (p.mode == kModePi && p.alpha != nullptr && hvalid) {
    const float a = p.alpha[(size_t)b * p.Hq + hq];
    bias_loc = __log2f(a);
    bias_skip = __log2f(1.0f - a);
  }

  // Query fragment (B operand): column t = query head of the group.
  constexpr int NQF = D / 4;
  float qf[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) qf[kk] = hvalid ? Qp[4 * kk + G] : 0.f;

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
  float m_run = kNegBig, l_run = 0.f;

  // Online softmax over the 4 score rows this lane holds (rows r0 + 4G + jj,
  // head column t); returns them as probabilities.
  auto softmax_step = [&](f32x4 s, int r0) -> f32x4 {
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int rr = r0 + 4 * G + jj;
      s[jj] = rr < sr.count ? fmaf(s[jj], p.scale_log2, sr.skip_row(rr) ? bias_skip : bias_loc) : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = mx;
    if (__any(m_new > m_run + kTau)) {
      const float mr = fmaxf(m_run, m_new);
      const float f = fast_exp2(m_run - mr);
      l_run *= f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= f;
      m_run = mr;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      s[jj] = fast_exp2(s[jj] - m_run);
      l_run += s[jj];
    }
    return s;
  };

  for (int r0 = 16 * wave; r0 < sr.count; r0 += 16 * kWaves) {
    const bool rvalid = r0 + t < sr.count;
    const int prow = sr.pos(min(r0 + t, sr.count - 1));
    f32x4 s = f32x4{};
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk) {
      const float a = rvalid ? (float)Kp[(size_t)prow * D + 4 * kk + G] : 0.f;
      s = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[kk], s, 0, 0, 0);
    }
    s = softmax_step(s, r0);
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

  // ---- merge the four waves pairwise through LDS (every lane keeps its C
  // layout: head column t, dims 16*db + 4G + jj), then write the split ------
  l_run += wave_shfl_xor(l_run, 16);
  l_run += wave_shfl_xor(l_run, 32);
  auto publish = [&](int slot) {
    f32x4 *A = (f32x4 *)(smem + slot * kSlotBytes);
    float *ML = (float *)(A + NDB * 64);
#pragma unroll
    for (int db = 0; db < NDB; ++db) A[db * 64 + lane] = acc[db];
    ML[lane] = m_run;
    ML[64 + lane] = l_run;
  };
  auto absorb = [&](int slot) {
    const f32x4 *A = (const f32x4 *)(smem + slot * kSlotBytes);
    const float *ML = (const float *)(A + NDB * 64);
    const float m1 = ML[lane], l1 = ML[64 + lane];
    const float mn = fmaxf(m_run, m1);
    const float f0 = fast_exp2(m_run - mn), f1 = fast_exp2(m1 - mn);
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = acc[db] * f0 + A[db * 64 + lane] * f1;
    l_run = l_run * f0 + l1 * f1;
    m_run = mn;
  };
  __syncthreads();                    // every wave is done streaming
  if (wave >= 2) publish(wave - 2);
  __syncthreads();
  if (wave < 2) absorb(wave);
  __syncthreads();
  if (wave == 1) publish(0);
  __syncthreads();
  if (wave != 0) return;
  absorb(0);
  if (!hvalid) return;
  float *wp = p.ws + (((size_t)b * p.Hq + hq) * p.nsplit + split) * ws_stride<D>();
  if (G == 0) {
    wp[0] = len_ok ? m_run : NAN;
    wp[1] = l_run;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) *(f32x4 *)(wp + 4 + 16 * db + 4 * G) = acc[db];
}

// ---------------------------------------------------------------------------
// bf16 decode.  Scores as in the fp32 kernel (S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16, query heads of the group as columns), but O is
// accumulated with v_mfma_f32_4x4x4bf16_1k, whose 16 independent 4x4 blocks
// fit a GQA group of 4 query heads exactly:
//   block b (lanes 4b..4b+3):  O_b[head i][dim 4b+j] += P[head i][row k] V[row k][dim 4b+j]
//   A: lane 4b+i holds P[head i][rows 4q..4q+3] (the same for every block),
//   B: lane 4b+j holds V[rows 4q..4q+3][dim 4b+j] (a transposed LDS read),
//   C: lane 4b+j, register i holds O[head i][dim 4b+j].
// One instruction covers 64 dims of 4 heads, so the accumulator is 4 registers
// per 64 dims and 4 heads (instead of 16 per 64 dims with 16 head columns), and
// more waves fit per SIMD.  HC4 = 4-head chunks per workgroup (heads of the
// group handled by one workgroup, up to 16).
// ---------------------------------------------------------------------------
template <int D, int HC4, int LAYOUT>
__global__ __launch_bounds__(256) void decode_bf16_kernel(Params p) {
  // Per-wave slabs of the group's 16 rows.  K: row stride 16 bytes mod 256,
  // so the 16 rows of an A-fragment read hit distinct banks.  V: row stride
  // 64 bytes mod 256, so the 4 rows x 2 column groups of a 32-lane transposed
  // read cover all 64 banks once.
  constexpr int LDK = D + 8;
  constexpr int LD = D == 64 ? 96 : 160;
  constexpr int NH = D / 64;          // 64-dim halves of O
  constexpr int NQF = D / 32;
  constexpr int NHD = 4 * HC4;        // heads per workgroup
  constexpr int kWaveSlab = 16 * (LDK + LD) * 2;
  constexpr int kSlabBytes = kWaves * kWaveSlab;
  constexpr int kSlotBytes = HC4 * NH * 64 * 16 + 2 * NHD * 4;
  constexpr int kSmem = kSlabBytes > 2 * kSlotBytes ? kSlabBytes : 2 * kSlotBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = lane >> 4, t = lane & 15;
  // One split per workgroup, or (walk_splits) every split in turn with the
  // running softmax state carried across them.  Contiguous and ring caches walk
  // the window rows as one split (a paged split's pages must fit one table
  // entry per lane).
  const int split = p.walk_splits ? 0 : blockIdx.x;
  const bool merged = p.walk_splits && LAYOUT != kCachePaged;
  const int g = blockIdx.y / p.hchunks, hc = blockIdx.y % p.hchunks;
  const int b = blockIdx.z;
  const int len = p.lens[b];
  // a ring cache holds any number of written tokens (the last R of them)
  bool len_ok = len >= 1 && (LAYOUT == kCacheRing || len <= p.Lmax);
  const int i = len_ok ? len - 1 : 0;
  const int head = 16 * hc + t;               // score column t = head of the group
  const bool hvalid = head < p.grp && t < NHD;
  const int hq = g * p.grp + head;
  const size_t kvoff = LAYOUT == kCachePaged ? 0
                       : (size_t)(b * p.Hkv + g) * (LAYOUT == kCacheRing ? p.R : p.Lmax) * D;
  const bf16 *Kp = (const bf16 *)p.kc + kvoff;
  const bf16 *Vp = (const bf16 *)p.vc + kvoff;
  const bf16 *Qp = (const bf16 *)p.q + ((size_t)b * p.Hq + hq) * D;

  SplitRows sr = merged ? window_rows(p, i) : split_rows(p, i, split);
  if (!len_ok) sr.count = 0;
  bool bad_page;
  RowMap<LAYOUT> rm = make_rowmap<LAYOUT>(p, sr, b, g, lane, bad_page);
  if (bad_page) {   // an unmapped page: NaN output, no cache access
    len_ok = false;
    sr.count = 0;
  }
  const int fallback = LAYOUT == kCacheContig ? i : 0;   // an in-range physical row

  float bias_loc = 0.f, bias_skip = 0.f;   // log2 priors of local and skip keys
  if (p.mode == kModePi && p.alpha != nullptr && p.opt.gate_w == nullptr && hvalid) {
    const float a = p.alpha[(size_t)b * p.Hq + hq];
    bias_loc = __log2f(a);
    bias_skip = __log2f(1.0f - a);
  }

  bf16x8 qf[NQF];
#pragma unroll
  for (int kk = 0; kk < NQF; ++kk) qf[kk] = hvalid ? *(const bf16x8 *)(Qp + 32 * kk + 8 * G) : bf16x8{};
  float sl2 = p.scale_log2;   // score scale of head column t (log2 units), set below
  f32x4 acc[HC4][NH];
#pragma unroll
  for (int c4 = 0; c4 < HC4; ++c4)
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) acc[c4][hh] = f32x4{};
  float m_run = kNegBig, l_run = 0.f;   // score layout: head t

  bf16 *ks = (bf16 *)(smem + wave * kWaveSlab);
  bf16 *vs = ks + 16 * LDK;
  auto consume = [&](const Group<D> &cur, int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < Group<D>::NC; ++u) {
      const int ci = lane + 64 * u, row = ci / (D / 8), col = (ci % (D / 8)) * 8;
      *(u32x4 *)(ks + row * LDK + col) = cur.k[u];
      *(u32x4 *)(vs + row * LD + col) = cur.v[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // S^T = K Q^T: A fragment = row t, dims 32kk + 8G .. +7.
    f32x4 s = f32x4{};
    float kss = 0.f;
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk) {
      const bf16x8 ka = *(const bf16x8 *)(ks + t * LDK + 32 * kk + 8 * G);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk], s, 0, 0, 0);
      if (p.opt.cosine) {   // |k|^2 with packed bf16 dot products
        const bf16x2 x0 = __builtin_shufflevector(ka, ka, 0, 1), x1 = __builtin_shufflevector(ka, ka, 2, 3);
        const bf16x2 x2 = __builtin_shufflevector(ka, ka, 4, 5), x3 = __builtin_shufflevector(ka, ka, 6, 7);
        kss = __builtin_amdgcn_fdot2_f32_bf16(x0, x0, kss, false);
        kss = __builtin_amdgcn_fdot2_f32_bf16(x1, x1, kss, false);
        kss = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, kss, false);
        kss = __builtin_amdgcn_fdot2_f32_bf16(x3, x3, kss, false);
      }
    }
    if (p.opt.cosine) {   // 1/|k| of row t, then of the rows 4G + jj this lane scores
      kss += wave_shfl_xor(kss, 16);
      kss += wave_shfl_xor(kss, 32);
      const float rk = rsqrtf(kss);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) s[jj] *= __shfl(rk, 4 * G + jj, 64);
    }
    // ---- online softmax per head column (rows r0 + 4G + jj) ----------------
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int rr = r0 + 4 * G + jj;
      s[jj] = rr < sr.count ? fmaf(s[jj], sl2, sr.skip_row(rr) ? bias_skip : bias_loc) : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = mx;
    if (__any(m_new > m_run + kTau)) {
      const float mr = fmaxf(m_run, m_new);
      const float f = fast_exp2(m_run - mr);
      l_run *= f;
      m_run = mr;
#pragma unroll
      for (int c4 = 0; c4 < HC4; ++c4)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float fh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), 4 * c4 + ii));
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) acc[c4][hh][ii] *= fh;
        }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      s[jj] = fast_exp2(s[jj] - m_run);
      l_run += s[jj];
    }
    bf16x4 pb;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) pb[jj] = (bf16)s[jj];
    const int2 pw = __builtin_bit_cast(int2, pb);
    // ---- O += P V over the 4 row quads of the group --------------------------
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4 vb[NH];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const bf16 *src = vs + (4 * q + (t >> 2)) * LD + 16 * G + 64 * hh + 4 * (t & 3);
        vb[hh] = as_bf16x4(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)src));
      }
#pragma unroll
      for (int c4 = 0; c4 < HC4; ++c4) {
        // P[head 4c4 + (lane & 3)][rows 4q..4q+3] lives in score lane 16q + 4c4 + (lane & 3).
        const int src_lane = 16 * q + 4 * c4 + (lane & 3);
        int2 a2;
        a2.x = __builtin_amdgcn_ds_bpermute(4 * src_lane, pw.x);
        a2.y = __builtin_amdgcn_ds_bpermute(4 * src_lane, pw.y);
        const bf16x4 pa = __builtin_bit_cast(bf16x4, a2);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) acc[c4][hh] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pa, vb[hh], acc[c4][hh], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Rows are streamed in 16-row groups, wave w taking groups w, w+4, ...; one
  // group's loads stay in flight while the previous group is consumed.
  constexpr int kStep = 16 * kWaves;
  Group<D> ring[kRing];
#pragma unroll
  for (int j = 0; j + 1 < kRing; ++j) ring[j] = load_group<D>(Kp, Vp, rm, 16 * wave + j * kStep, lane, fallback);
  // Cosine scale and query-driven gate, computed while the first rows load
  // (their global reads would otherwise delay the row stream).
  if (p.opt.cosine) {
    // lane (G, t) holds dims 32kk + 8G .. +7 of head t; the groups G hold the row
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)qf[kk][e], (float)qf[kk][e], ss);
    ss += wave_shfl_xor(ss, 16);
    ss += wave_shfl_xor(ss, 32);
    sl2 *= hvalid ? rsqrtf(ss) : 0.f;
  }
  if (p.opt.gate_w != nullptr && p.mode == kModePi) {   // alpha = sigmoid(gate network of q)
    float z = 0.f;
    if (p.opt.gate_hidden > 0) {
      // Two layers, ReLU hidden layer.  The columns are different heads: one
      // pass of the network per head of this workgroup, each keeping its column.
#pragma unroll
      for (int hd = 0; hd < NHD; ++hd) {
        if (16 * hc + hd >= p.grp) break;
        const GateMlp gm = make_gate(p.opt.gate_w, p.opt.gate_b, p.opt.gate_w2, p.opt.gate_b2, p.opt.gate_hidden,
                                     g * p.grp + 16 * hc + hd, D);
        const float zh = gate_mlp_logit_16<D>(qf, gm, lane);
        if (t == hd) z = zh;
      }
    } else {
      const float *w = p.opt.gate_w + (size_t)(hvalid ? hq : 0) * D + 8 * G;
      f32x4 wv[NQF][2];
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk) {
        wv[kk][0] = *(const f32x4 *)(w + 32 * kk);
        wv[kk][1] = *(const f32x4 *)(w + 32 * kk + 4);
      }
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) z = fmaf((float)qf[kk][e], wv[kk][e >> 2][e & 3], z);
      z += wave_shfl_xor(z, 16);
      z += wave_shfl_xor(z, 32);
      z += p.opt.gate_b[hvalid ? hq : 0];
    }
    if (hvalid) {   // log2 alpha and log2(1 - alpha), overflow-free
      const float l1 = __log2f(1.0f + fast_exp2(-fabsf(z) * kLog2e));
      bias_loc = (z >= 0.f ? 0.f : z * kLog2e) - l1;
      bias_skip = (z <= 0.f ? 0.f : -z * kLog2e) - l1;
    }
  }

  const int nwalk = merged ? 2 : p.walk_splits ? p.nsplit : 1;
  for (int sidx = 0; sidx < nwalk; ++sidx) {
    if (sidx > 0) {   // next split of the walk: its rows, row map and first group
      sr = split_rows(p, i, merged ? p.n_wsplit : sidx);
      if (!len_ok) sr.count = 0;
      rm = make_rowmap<LAYOUT>(p, sr, b, g, lane, bad_page);
      if (bad_page) {
        len_ok = false;
        sr.count = 0;
      }
#pragma unroll
      for (int j = 0; j + 1 < kRing; ++j) ring[j] = load_group<D>(Kp, Vp, rm, 16 * wave + j * kStep, lane, fallback);
    }
    for (int r0 = 16 * wave; r0 < sr.count; r0 += kRing * kStep) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        ring[(j + kRing - 1) % kRing] = load_group<D>(Kp, Vp, rm, r0 + (j + kRing - 1) * kStep, lane, fallback);
        if (r0 + j * kStep < sr.count) consume(ring[j], r0 + j * kStep);
      }
    }
  }

  // ---- per-head state (uniform), then merge the four waves pairwise --------
  l_run += wave_shfl_xor(l_run, 16);
  l_run += wave_shfl_xor(l_run, 32);
  float m_h[NHD], l_h[NHD];
#pragma unroll
  for (int k = 0; k < NHD; ++k) {
    m_h[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_run), k));
    l_h[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_run), k));
  }
  auto publish = [&](int slot) __attribute__((always_inline)) {
    f32x4 *A = (f32x4 *)(smem + slot * kSlotBytes);
    float *ML = (float *)(A + HC4 * NH * 64);
#pragma unroll
    for (int c4 = 0; c4 < HC4; ++c4)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) A[(c4 * NH + hh) * 64 + lane] = acc[c4][hh];
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < NHD; ++k) {
        ML[2 * k] = m_h[k];
        ML[2 * k + 1] = l_h[k];
      }
    }
  };
  auto absorb = [&](int slot) __attribute__((always_inline)) {
    const f32x4 *A = (const f32x4 *)(smem + slot * kSlotBytes);
    const float *ML = (const float *)(A + HC4 * NH * 64);
#pragma unroll
    for (int c4 = 0; c4 < HC4; ++c4)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int k = 4 * c4 + ii;
        const float m1 = ML[2 * k], l1 = ML[2 * k + 1];
        const float mn = fmaxf(m_h[k], m1);
        const float f0 = fast_exp2(m_h[k] - mn), f1 = fast_exp2(m1 - mn);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) acc[c4][hh][ii] = acc[c4][hh][ii] * f0 + A[(c4 * NH + hh) * 64 + lane][ii] * f1;
        l_h[k] = l_h[k] * f0 + l1 * f1;
        m_h[k] = mn;
      }
  };
  __syncthreads();                    // the V slabs are free
  if (wave >= 2) publish(wave - 2);
  __syncthreads();
  if (wave < 2) absorb(wave);
  __syncthreads();
  if (wave == 1) publish(0);
  __syncthreads();
  if (wave != 0) return;
  absorb(0);
  if (p.walk_splits) {   // every split done: normalise, gate and write o
#pragma unroll
    for (int c4 = 0; c4 < HC4; ++c4)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int hd = 16 * hc + 4 * c4 + ii;
        if (hd >= p.grp) continue;
        const size_t row = (size_t)b * p.Hq + g * p.grp + hd;
        const float inv = len_ok ? 1.0f / l_h[4 * c4 + ii] : NAN;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          float o = acc[c4][hh][ii] * inv;
          if (p.opt.out_gate != nullptr) {
            const unsigned short gu = ((const unsigned short *)p.opt.out_gate)[row * D + lane + 64 * hh];
            o *= sigmoid_fast(bf16_to_f32(gu));
          }
          ((unsigned short *)p.o)[row * D + lane + 64 * hh] = f32_to_bf16_bits(o);
        }
      }
    return;
  }
  // ---- write this split's partial state: lane l holds dims l + 64hh ------------
#pragma unroll
  for (int c4 = 0; c4 < HC4; ++c4)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int hd = 16 * hc + 4 * c4 + ii;
      if (hd >= p.grp) continue;
      float *wp = p.ws + (((size_t)b * p.Hq + g * p.grp + hd) * p.nsplit + split) * ws_stride<D>();
      if (lane == 0) {
        wp[0] = len_ok ? m_h[4 * c4 + ii] : NAN;
        wp[1] = l_h[4 * c4 + ii];
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) wp[4 + lane + 64 * hh] = acc[c4][hh][ii];
    }
}

// Merge the split partials of one (sequence, query head) and normalise: one
// thread per output dimension, an online log-sum-exp merge over the splits.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(Params p) {
  const int row = blockIdx.x;  // b*Hq + hq
  const int dim = threadIdx.x;
  const float *wp = p.ws + (size_t)row * p.nsplit * ws_stride<D>();
  float m = kNegBig, l = 0.f, a = 0.f;
  bool bad = false;
#pragma unroll 4
  for (int s = 0; s < p.nsplit; ++s) {
    const float *e = wp + s * ws_stride<D>();
    const float ms = e[0], ls = e[1], as = e[4 + dim];
    bad |= ms != ms;
    const float mn = fmaxf(m, ms);
    const float f0 = fast_exp2(m - mn), f1 = fast_exp2(ms - mn);
    l = l * f0 + ls * f1;
    a = a * f0 + as * f1;
    m = mn;
  }
  float o = bad ? NAN : a / l;
  if constexpr (sizeof(T) == 2) {
    if (p.opt.out_gate != nullptr) {   // output gate o * sigmoid(g)
      const unsigned short gu = ((const unsigned short *)p.opt.out_gate)[(size_t)row * D + dim];
      o *= sigmoid_fast(bf16_to_f32(gu));
    }
  }
  T *op = (T *)p.o + (size_t)row * D + dim;
  if constexpr (sizeof(T) == 2) *(unsigned short *)op = f32_to_bf16_bits(o);
  else *op = o;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
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
  p.opt = a.opt;
  p.scale_log2 = kLog2e * (a.opt.score_scale > 0.f ? a.opt.score_scale : 1.0f / sqrtf((float)D));
  p.R = a.R; p.page_shift = a.page_shift; p.num_pages = a.num_pages; p.max_pages = a.max_pages; p.table = a.table;
  // Each (sequence, KV head, head chunk) workgroup walks all of its splits and
  // writes o itself when those workgroups fill at least three quarters of the
  // compute units in their last round (one workgroup then streams its rows
  // at a fraction of a CU's bandwidth, so a round that leaves many CUs idle
  // loses to the split plan).  Otherwise: one workgroup per split, and the
  // combine kernel merges them.
  p.walk_splits = 0;
  if constexpr (sizeof(T) == 2) {
    const long long wgs = (long long)a.B * a.Hkv * p.hchunks, cus = cu_count();
    p.walk_splits = 4 * wgs >= 3 * cus * ((wgs + cus - 1) / cus);
  }
  const dim3 grid(p.walk_splits ? 1 : p.nsplit, a.Hkv * p.hchunks, a.B);
  if constexpr (sizeof(T) == 2) {
    const int heads = p.grp < 16 ? p.grp : 16;   // heads per workgroup
    const int hc4 = heads <= 4 ? 1 : heads <= 8 ? 2 : 4;
#define SA_DECODE_LAUNCH(L)                                                                  \
  if (hc4 == 1) hipLaunchKernelGGL((decode_bf16_kernel<D, 1, L>), grid, dim3(256), 0, s, p); \
  else if (hc4 == 2) hipLaunchKernelGGL((decode_bf16_kernel<D, 2, L>), grid, dim3(256), 0, s, p); \
  else hipLaunchKernelGGL((decode_bf16_kernel<D, 4, L>), grid, dim3(256), 0, s, p);
    if (a.layout == kCacheRing) {
      SA_DECODE_LAUNCH(kCacheRing)
    } else if (a.layout == kCachePaged) {
      SA_DECODE_LAUNCH(kCachePaged)
    } else {
      SA_DECODE_LAUNCH(kCacheContig)
    }
#undef SA_DECODE_LAUNCH
  } else {
    if (a.layout != kCacheContig) return hipErrorInvalidValue;   // fp32: contiguous caches only
    hipLaunchKernelGGL((decode_f32_kernel<D>), grid, dim3(256), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.walk_splits) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.B * a.Hq), dim3(D), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.dtype == kBF16) return a.d == 64 ? launch_t<bf16, 64>(a, s) : launch_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_t<float, 64>(a, s) : launch_t<float, 128>(a, s);
}

}  // namespace sa
