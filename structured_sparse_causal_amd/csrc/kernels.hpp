// kernels.hpp -- host-side launch interface between the C ABI (api.hip) and the
// gfx950 kernels.  Internal to libsparse_attn; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace sa {

enum { kModePi = 0, kModeWindow = 1, kModeEcp = 2, kModeWindowBidir = 3, kModeSsplit = 4, kModeEcpFull = 5 };
enum { kF32 = 0, kBF16 = 1 };

// Prefill: query block of 128 rows per workgroup; key tiles of 64 rows (the
// bf16 kernel at d = 128 uses 32-row tiles; see prefill.hip).
constexpr int kPrefillBM = 128;
constexpr int kPrefillBN = 64;

// Fused gate and epilogue options (all off when zero / null):
//   score_scale > 0 replaces 1/sqrt(d); cosine: scores are scale * cos(q, k)
//   (the key rows given to the kernels are already L2-normalised; the query's
//   norm is taken in-kernel); the gate network on the query (PI) for head
//   h = (gate_bh0 + local (batch, head) index) % gate_hq (the prefill and the
//   skip pass take the one-layer gate in-kernel and the two-layer network's
//   alpha from a pre-pass; the decode evaluates both in-kernel):
//   gate_hidden = 0: gate_w [Hq][d] / gate_b [Hq], alpha =
//   sigmoid(<gate_w[h], q_i> + gate_b[h]); gate_hidden = H in [1, 32]:
//   gate_w [Hq][H][d], gate_b [Hq][H], gate_w2 [Hq][H], gate_b2 [Hq], alpha =
//   sigmoid(sum_u gate_w2[h][u] relu(<gate_w[h][u], q_i> + gate_b[h][u]) +
//   gate_b2[h]); out_gate: output o * sigmoid(out_gate), same layout and dtype
//   as o.
struct FusedOpts {
  float score_scale;
  int cosine;
  const float *gate_w, *gate_b;
  int gate_bh0, gate_hq;
  const void *out_gate;
  int gate_hidden;
  const float *gate_w2, *gate_b2;
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float *alpha;   // [B,Hq,N] or nullptr (PI priors)
  void *o;
  const float *skip_ml; // [B*Hq*N][2] (running max in log2 units, sum) or nullptr
  const void *skip_acc; // [B*Hq*N][d] unnormalised skip accumulators (I/O dtype) or nullptr
  float *lse;           // [B*Hq*N] natural-log row normaliser (training forward) or nullptr
  int B, Hq, Hkv, N, d, dtype;
  int mode, k_win, seg;
  int skip_first;       // first query position that has a skip key (PI), else N
  FusedOpts opt;
};

struct SkipArgs {
  const void *q, *k, *v;
  const float *alpha;   // [B,Hq,N]
  float *ml;            // [B*Hq*N][2]
  void *acc;            // [B*Hq*N][d] in the I/O dtype
  int B, Hq, Hkv, N, d, dtype;
  int pi, M, m_min;     // skip offsets m*pi for m in [m_min, M]
  FusedOpts opt;        // score_scale, cosine, gate (out_gate unused)
};

struct DecodeArgs {
  const void *q, *kc, *vc;
  const int *lens;
  const float *alpha;   // [B,Hq] or nullptr
  void *o;
  float *ws;            // [B*Hq][nsplit][d+4]: max, sum, 2 pad, accumulator
  int B, Hq, Hkv, Lmax, d, dtype;
  int mode, k_win, pi, M, seg, m_min;
  int n_wsplit, chunk, nsplit;   // window splits, rows per window split, n_wsplit + 1
  // Cache layout: kCacheContig kc/vc [B,Hkv,Lmax,d]; kCacheRing kc/vc [B,Hkv,R,d]
  // with position p in slot p mod R; kCachePaged kc/vc [num_pages,Hkv,P,d] with
  // block table [B][max_pages] (P = 1 << page_shift, Lmax = max_pages * P).
  int layout, R, page_shift, num_pages, max_pages;
  const int *table;
  FusedOpts opt;        // bf16 only (gate_bh0 = 0, gate_hq = Hq)
};
enum { kCacheContig = 0, kCacheRing = 1, kCachePaged = 2 };

struct BwdArgs {
  const void *q, *k, *v, *o, *dO;   // bf16
  const float *alpha, *lse;         // [B,Hq,N]
  void *dq, *dk, *dv;               // bf16
  float *dalpha;                    // [B,Hq,N] or nullptr
  float *Dv, *cv;                   // workspace [B*Hq*N (+pad)]
  int skips;                        // pi-Attention with skip keys (skip kernels after the walks)
  int B, Hq, Hkv, N, d;
  int mode, k_win, pi, M, m_min, seg;
  float score_scale;                // 0: 1/sqrt(d)
  const void *out_gate;             // output gate g (bf16, like o) or nullptr
  void *dgate;                      // dL/dg (bf16) when out_gate is given
  void *dO_gated;                   // workspace [B*Hq*N][d] bf16: dO * sigmoid(g)
};
// alpha [BH][N] of every query row from the two-layer gate network in o (head = bh % Hq).
hipError_t launch_gate_alpha(const void *q, float *alpha, int BH, int Hq, int N, int d, int dtype, const FusedOpts &o,
                             hipStream_t s);
hipError_t launch_normalize_rows(const void *src, void *dst, long long rows, int d, int dtype, hipStream_t s);

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s);
hipError_t launch_skip(const SkipArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

}  // namespace sa
