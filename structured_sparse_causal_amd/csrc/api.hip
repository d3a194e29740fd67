// api.hip -- the C ABI of libsparse_attn (declared in include/sparse_attn.h):
// argument validation on the host (before any HIP call), workspace sizing,
// and the launch sequence on the caller's stream.  No allocation, no
// synchronisation, no global state apart from the per-thread error text.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "sparse_attn.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return code;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Common checks of the mode parameters.  Returns SA_OK or an error code.
int check_mode(int mode, int k_win, int pi, int M, int seg) {
  if (mode == SA_MODE_ECP || mode == SA_MODE_SSPLIT || mode == SA_MODE_ECP_FULL) {
    if (seg <= 0) return fail(SA_ERR_INVALID, "segment modes need seg >= 1");
    return SA_OK;
  }
  if (mode != SA_MODE_PI && mode != SA_MODE_WINDOW && mode != SA_MODE_WINDOW_BIDIR)
    return fail(SA_ERR_INVALID, "unknown mode");
  if (k_win < 0) return fail(SA_ERR_INVALID, "k_win must be >= 0");
  if (mode == SA_MODE_PI) {
    if (M < 0) return fail(SA_ERR_INVALID, "M must be >= 0");
    if (M > 0 && pi <= 0) return fail(SA_ERR_INVALID, "pi must be >= 1 when M > 0");
  }
  return SA_OK;
}

int check_shape(int dtype, int d) {
  if (dtype != SA_DTYPE_F32 && dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  return SA_OK;
}

size_t elem_size(int dtype) { return dtype == SA_DTYPE_BF16 ? 2 : 4; }

// Smallest m with m*pi > k_win: the first skip offset lying below the window.
long long skip_m_min(int k_win, int pi) { return (long long)k_win / pi + 1; }

// True when some query of a length-N sequence has a skip key below its window.
bool has_skips(int mode, int k_win, int pi, int M, int N) {
  if (mode != SA_MODE_PI || M <= 0) return false;
  const long long mm = skip_m_min(k_win, pi);
  return mm <= M && mm * (long long)pi <= (long long)N - 1;
}

// pi-Attention with skip keys runs as (skip pass, prefill) pairs over chunks of
// whole GQA groups of (batch, head) slices.  The workspace holds one chunk's
// skip state (an (m, l) pair and a d-wide accumulator per query row) and is
// capped at kChunkBytes, so it stays resident in the 256 MB last-level cache
// between the two launches and does not grow with B * Hq.  Chunks are
// balanced: a short last chunk would leave most of the GPU idle.
constexpr size_t kChunkBytes = (size_t)128 << 20;

int fwd_chunk_heads(int B, int Hq, int Hkv, int N, int d, int dtype) {
  const int grp = Hq / Hkv;
  const size_t per_group = (size_t)grp * N * (2 * sizeof(float) + (size_t)d * elem_size(dtype));
  size_t fit = kChunkBytes / per_group;
  if (fit < 1) fit = 1;
  const size_t total_groups = (size_t)B * Hkv;
  const size_t nchunks = (total_groups + fit - 1) / fit;
  const size_t groups = (total_groups + nchunks - 1) / nchunks;
  return (int)(groups * grp);
}

struct FwdLayout {
  size_t ml_off, acc_off, total;
};

FwdLayout fwd_layout(int heads, int N, int d, int dtype) {
  FwdLayout L;
  const size_t rows = (size_t)heads * N;
  L.ml_off = 0;
  L.acc_off = round_up(rows * 2 * sizeof(float), 256);
  L.total = L.acc_off + round_up(rows * (size_t)d * elem_size(dtype), 256);
  return L;
}

int fwd_validate(const void *q, const void *k, const void *v, const float *alpha, void *o, int B, int Hq,
                 int Hkv, int N, int d, int dtype, int mode, int k_win, int pi, int M, int seg,
                 bool gate_from_q = false) {
  int rc = check_shape(dtype, d);
  if (rc != SA_OK) return rc;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return fail(SA_ERR_INVALID, "B, Hq, Hkv and N must be >= 1");
  if (Hq % Hkv != 0) return fail(SA_ERR_INVALID, "Hq must be a multiple of Hkv");
  rc = check_mode(mode, k_win, pi, M, seg);
  if (rc != SA_OK) return rc;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return fail(SA_ERR_INVALID, "null tensor pointer");
  if (mode == SA_MODE_PI && M > 0 && alpha == nullptr && !gate_from_q)
    return fail(SA_ERR_INVALID, "alpha is required for PI mode with M > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(alpha, 4))
    return fail(SA_ERR_INVALID, "misaligned tensor (q/k/v/o need 16 bytes, alpha 4)");
  const long long rows = (long long)B * Hq * N;
  const long long blocks = (long long)B * Hq * ((N + sa::kPrefillBM - 1) / sa::kPrefillBM);
  if (rows >= (1LL << 31) || blocks >= (1LL << 31) || (long long)N * d >= (1LL << 31))
    return fail(SA_ERR_INVALID, "problem too large for 32-bit row indexing");
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)rows * d * es, nkv = (size_t)B * Hkv * N * d * es;
  const size_t na = (mode == SA_MODE_PI && alpha) ? (size_t)rows * sizeof(float) : 0;
  if (overlap(o, nq, q, nq) || overlap(o, nq, k, nkv) || overlap(o, nq, v, nkv) || overlap(o, nq, alpha, na))
    return fail(SA_ERR_INVALID, "output overlaps an input");
  return SA_OK;
}

}  // namespace

extern "C" {

size_t sparse_attn_fwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype, int mode, int k_win,
                                      int pi, int M, int seg) {
  if (check_shape(dtype, d) != SA_OK || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || Hq % Hkv != 0 ||
      check_mode(mode, k_win, pi, M, seg) != SA_OK)
    return 0;
  if (!has_skips(mode, k_win, pi, M, N)) return 0;
  return fwd_layout(fwd_chunk_heads(B, Hq, Hkv, N, d, dtype), N, d, dtype).total;
}

}  // extern "C"

namespace {

// Options of the *_ex entry points, as the kernels take them.
sa::FusedOpts fused_opts(const sa_options *opt, int Hq) {
  sa::FusedOpts f;
  f.score_scale = opt != nullptr ? opt->score_scale : 0.f;
  f.cosine = opt != nullptr && opt->cosine != 0;
  f.gate_w = opt != nullptr ? opt->gate_w : nullptr;
  f.gate_b = opt != nullptr ? opt->gate_b : nullptr;
  f.gate_bh0 = 0;
  f.gate_hq = Hq;
  f.out_gate = opt != nullptr ? opt->out_gate : nullptr;
  f.gate_hidden = opt != nullptr ? opt->gate_hidden : 0;
  f.gate_w2 = opt != nullptr ? opt->gate_w2 : nullptr;
  f.gate_b2 = opt != nullptr ? opt->gate_b2 : nullptr;
  return f;
}

int check_opts(const sa::FusedOpts &f, int mode) {
  if (!(f.score_scale >= 0.f) || f.score_scale > 3.0e38f) return fail(SA_ERR_INVALID, "score_scale must be finite and >= 0");
  if ((f.gate_w == nullptr) != (f.gate_b == nullptr)) return fail(SA_ERR_INVALID, "gate_w and gate_b go together");
  if (f.gate_w != nullptr && mode != SA_MODE_PI) return fail(SA_ERR_INVALID, "the query-driven gate is a PI-mode option");
  if (f.gate_hidden < 0 || f.gate_hidden > 32) return fail(SA_ERR_INVALID, "gate_hidden must lie in [0, 32]");
  if (f.gate_hidden > 0 && (f.gate_w == nullptr || f.gate_w2 == nullptr || f.gate_b2 == nullptr))
    return fail(SA_ERR_INVALID, "the gate network (gate_hidden > 0) needs gate_w, gate_b, gate_w2 and gate_b2");
  if (f.gate_hidden == 0 && (f.gate_w2 != nullptr || f.gate_b2 != nullptr))
    return fail(SA_ERR_INVALID, "gate_w2 / gate_b2 given without gate_hidden");
  if (!aligned(f.gate_w, 16) || !aligned(f.gate_b, 4) || !aligned(f.gate_w2, 4) || !aligned(f.gate_b2, 4) ||
      !aligned(f.out_gate, 16))
    return fail(SA_ERR_INVALID, "misaligned option tensor");
  return SA_OK;
}

// Bytes of the L2-normalised key copy that cosine scores read.
size_t khat_bytes(const sa::FusedOpts &f, int B, int Hkv, int N, int d, int dtype) {
  return f.cosine ? round_up((size_t)B * Hkv * N * d * elem_size(dtype), 256) : 0;
}

// Bytes of the alpha rows the two-layer gate network's pre-pass writes (PI).
size_t gate_alpha_bytes(const sa::FusedOpts &f, int mode, int B, int Hq, int N) {
  return (f.gate_hidden > 0 && mode == SA_MODE_PI) ? round_up((size_t)B * Hq * N * sizeof(float), 256) : 0;
}

int fwd_impl(const void *q, const void *k, const void *v, const float *alpha, void *o, float *lse, int B, int Hq,
             int Hkv, int N, int d, int dtype, int mode, int k_win, int pi, int M, int seg, void *workspace,
             size_t workspace_bytes, void *stream, const sa::FusedOpts &fo = sa::FusedOpts{}) {
  g_err[0] = 0;
  int rc = fwd_validate(q, k, v, alpha, o, B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg,
                        fo.gate_w != nullptr && mode == SA_MODE_PI);
  if (rc != SA_OK) return rc;
  rc = check_opts(fo, mode);
  if (rc != SA_OK) return rc;
  // Every check happens here, before the first launch: an error return leaves
  // nothing enqueued.
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * Hq * N * d * es, nkv = (size_t)B * Hkv * N * d * es;
  const size_t nl = (size_t)B * Hq * N * sizeof(float);
  const size_t na = (mode == SA_MODE_PI && alpha != nullptr) ? nl : 0;
  const size_t ng = fo.out_gate != nullptr ? nq : 0;
  if (overlap(o, nq, fo.out_gate, ng)) return fail(SA_ERR_INVALID, "output overlaps out_gate");
  if (lse != nullptr) {
    if (!aligned(lse, 4)) return fail(SA_ERR_INVALID, "misaligned lse");
    if (overlap(lse, nl, q, nq) || overlap(lse, nl, o, nq) || overlap(lse, nl, k, nkv) || overlap(lse, nl, v, nkv) ||
        overlap(lse, nl, alpha, na) || overlap(lse, nl, fo.out_gate, ng))
      return fail(SA_ERR_INVALID, "lse overlaps a tensor");
  }
  // Workspace: [L2-normalised key copy (cosine scores)] [alpha from the gate
  // network (PI, two-layer gate)] [skip-key partial state (pi with skip keys)].
  const size_t kh = khat_bytes(fo, B, Hkv, N, d, dtype);
  const size_t ga = gate_alpha_bytes(fo, mode, B, Hq, N);
  const bool skips = has_skips(mode, k_win, pi, M, N);
  const int chunk = skips ? fwd_chunk_heads(B, Hq, Hkv, N, d, dtype) : 0;
  const FwdLayout L = skips ? fwd_layout(chunk, N, d, dtype) : FwdLayout{0, 0, 0};
  const size_t need = kh + ga + L.total;
  if (need > 0) {
    const size_t nh = fo.gate_hidden > 0 ? (size_t)fo.gate_hidden : 1;
    const size_t ngw = fo.gate_w ? (size_t)Hq * nh * d * 4 : 0, ngb = fo.gate_b ? (size_t)Hq * nh * 4 : 0;
    const size_t ngw2 = fo.gate_w2 ? (size_t)Hq * nh * 4 : 0, ngb2 = fo.gate_b2 ? (size_t)Hq * 4 : 0;
    if (workspace == nullptr || workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "workspace missing or smaller than the forward workspace size");
    if (!aligned(workspace, 256)) return fail(SA_ERR_INVALID, "workspace must be 256-byte aligned");
    if (overlap(workspace, need, q, nq) || overlap(workspace, need, k, nkv) || overlap(workspace, need, v, nkv) ||
        overlap(workspace, need, o, nq) || overlap(workspace, need, alpha, na) ||
        overlap(workspace, need, lse, lse != nullptr ? nl : 0) || overlap(workspace, need, fo.out_gate, ng) ||
        overlap(workspace, need, fo.gate_w, ngw) || overlap(workspace, need, fo.gate_b, ngb) ||
        overlap(workspace, need, fo.gate_w2, ngw2) || overlap(workspace, need, fo.gate_b2, ngb2))
      return fail(SA_ERR_INVALID, "workspace overlaps a tensor");
  }
  hipStream_t s = (hipStream_t)stream;
  sa::FusedOpts fk = fo;   // the options as the attention kernels take them
  if (ga > 0) {
    // alpha of every row from the gate network, once; the kernels then take it
    // as their alpha input
    float *wa = (float *)((char *)workspace + kh);
    hipError_t e = sa::launch_gate_alpha(q, wa, B * Hq, Hq, N, d, dtype, fo, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
    alpha = wa;
    fk.gate_w = fk.gate_b = fk.gate_w2 = fk.gate_b2 = nullptr;
    fk.gate_hidden = 0;
  }
  if (kh > 0) {
    hipError_t e = sa::launch_normalize_rows(k, workspace, (long long)B * Hkv * N, d, dtype, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
    k = workspace;   // scores read the normalised keys
  }
  workspace = (char *)workspace + kh + ga;
  sa::PrefillArgs pa;
  pa.q = q; pa.k = k; pa.v = v; pa.alpha = alpha; pa.o = o;
  pa.skip_ml = nullptr; pa.skip_acc = nullptr; pa.lse = lse;
  pa.B = B; pa.Hq = Hq; pa.Hkv = Hkv; pa.N = N; pa.d = d; pa.dtype = dtype;
  pa.mode = mode; pa.k_win = k_win; pa.seg = seg;
  pa.skip_first = N;
  pa.opt = fk;
  if (!skips) {
    hipError_t e = sa::launch_prefill(pa, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
    return SA_OK;
  }
  const long long mm = skip_m_min(k_win, pi);
  const int grp = Hq / Hkv;
  const size_t head_elems = (size_t)N * d;
  // A chunk of whole GQA groups is a contiguous range of (batch, head) slices;
  // the kernels see it as one batch of `n` query heads and n/grp KV heads.
  for (int bh0 = 0; bh0 < B * Hq; bh0 += chunk) {
    const int n = B * Hq - bh0 < chunk ? B * Hq - bh0 : chunk;
    sa::SkipArgs sk;
    sk.q = (const char *)q + (size_t)bh0 * head_elems * es;
    sk.k = (const char *)k + (size_t)(bh0 / grp) * head_elems * es;
    sk.v = (const char *)v + (size_t)(bh0 / grp) * head_elems * es;
    sk.alpha = alpha != nullptr ? alpha + (size_t)bh0 * N : nullptr;   // null with the query-driven gate
    sk.ml = (float *)((char *)workspace + L.ml_off);
    sk.acc = (char *)workspace + L.acc_off;
    sk.B = 1; sk.Hq = n; sk.Hkv = n / grp; sk.N = N; sk.d = d; sk.dtype = dtype;
    sk.pi = pi; sk.M = M; sk.m_min = (int)mm;
    sk.opt = fk;
    sk.opt.gate_bh0 = bh0;
    sk.opt.out_gate = nullptr;
    hipError_t e = sa::launch_skip(sk, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
    sa::PrefillArgs pc = pa;
    pc.q = sk.q; pc.k = sk.k; pc.v = sk.v; pc.alpha = sk.alpha;
    pc.o = (char *)o + (size_t)bh0 * head_elems * es;
    pc.B = 1; pc.Hq = n; pc.Hkv = n / grp;
    pc.skip_ml = sk.ml;
    pc.skip_acc = sk.acc;
    pc.skip_first = (int)(mm * pi);
    pc.lse = lse != nullptr ? lse + (size_t)bh0 * N : nullptr;
    pc.opt.gate_bh0 = bh0;
    if (fk.out_gate != nullptr) pc.opt.out_gate = (const char *)fk.out_gate + (size_t)bh0 * head_elems * es;
    e = sa::launch_prefill(pc, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
  }
  return SA_OK;
}

}  // namespace

extern "C" {

int sparse_attn_fwd(const void *q, const void *k, const void *v, const float *alpha, void *o, int B, int Hq,
                    int Hkv, int N, int d, int dtype, int mode, int k_win, int pi, int M, int seg,
                    void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, alpha, o, nullptr, B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg, workspace,
                  workspace_bytes, stream);
}

int sparse_attn_fwd_lse(const void *q, const void *k, const void *v, const float *alpha, void *o, float *lse,
                        int B, int Hq, int Hkv, int N, int d, int dtype, int mode, int k_win, int pi, int M,
                        int seg, void *workspace, size_t workspace_bytes, void *stream) {
  if (lse == nullptr) {
    g_err[0] = 0;
    return fail(SA_ERR_INVALID, "null lse pointer");
  }
  return fwd_impl(q, k, v, alpha, o, lse, B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg, workspace,
                  workspace_bytes, stream);
}

size_t sparse_attn_fwd_ex_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype, int mode, int k_win,
                                         int pi, int M, int seg, const sa_options *opt) {
  if (check_shape(dtype, d) != SA_OK || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || Hq % Hkv != 0 ||
      check_mode(mode, k_win, pi, M, seg) != SA_OK)
    return 0;
  const sa::FusedOpts fo = fused_opts(opt, Hq);
  return khat_bytes(fo, B, Hkv, N, d, dtype) + gate_alpha_bytes(fo, mode, B, Hq, N) +
         sparse_attn_fwd_workspace_size(B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg);
}

int sparse_attn_fwd_ex(const void *q, const void *k, const void *v, const float *alpha, void *o, float *lse,
                       int B, int Hq, int Hkv, int N, int d, int dtype, int mode, int k_win, int pi, int M,
                       int seg, const sa_options *opt, void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, alpha, o, lse, B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg, workspace,
                  workspace_bytes, stream, fused_opts(opt, Hq));
}

// Backward workspace: D_i and c_i per query row (+16 floats of padding for
// the 16-byte vector loads at the tail).  The skip-key contributions are
// added into dq, dk and dv in place, after the window walks.
struct BwdLayout {
  size_t dv_off, cv_off, total;
};

static BwdLayout bwd_layout(int B, int Hq, int N) {
  BwdLayout L;
  const size_t rows = (size_t)B * Hq * N;
  size_t at = 0;
  L.dv_off = at; at += round_up((rows + 16) * sizeof(float), 256);
  L.cv_off = at; at += round_up((rows + 16) * sizeof(float), 256);
  L.total = at;
  return L;
}

// Decode split plan: the window rows below the query (at most k_win, or
// 2*seg - 1 for ECP, never more than Lmax - 1) are cut into splits of about 256
// rows (a multiple of 64, the rows one pass of a 4-wave workgroup covers); one
// more split holds the query row and the skip keys.
static void decode_plan(int Lmax, int mode, int k_win, int pi, int seg, int *n_wsplit, int *chunk,
                        int *m_min) {
  long long range = mode == SA_MODE_ECP ? 2LL * seg : mode == SA_MODE_SSPLIT ? (long long)seg : (long long)k_win + 1;
  if (range > Lmax) range = Lmax;
  const long long below = range - 1;
  const int n = (int)((below + 255) / 256);
  long long c = n > 0 ? (below + n - 1) / n : 64;
  c = (c + 63) / 64 * 64;
  *n_wsplit = n;
  *chunk = (int)c;
  *m_min = (mode == SA_MODE_PI && pi > 0) ? (int)(skip_m_min(k_win, pi) < (1LL << 30) ? skip_m_min(k_win, pi) : (1LL << 30)) : 1;
}

size_t sparse_attn_decode_workspace_size(int B, int Hq, int Hkv, int Lmax, int d, int dtype, int mode, int k_win,
                                         int pi, int M, int seg) {
  if (check_shape(dtype, d) != SA_OK || B <= 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || Hq % Hkv != 0 ||
      check_mode(mode, k_win, pi, M, seg) != SA_OK || mode == SA_MODE_WINDOW_BIDIR || mode == SA_MODE_ECP_FULL)
    return 0;
  int nw, chunk, mm;
  decode_plan(Lmax, mode, k_win, pi, seg, &nw, &chunk, &mm);
  return round_up((size_t)B * Hq * (nw + 1) * (d + 4) * sizeof(float), 256);
}

namespace {

int scratch_for_current_device(void **out);
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;

// Shared body of the decode entry points.  Lplan: the largest position
// count the layout can hold (contiguous Lmax, ring R, paged max_pages * P);
// cache_bytes: bytes of each cache tensor (overlap checks).
int decode_impl(const void *q, const void *k_cache, const void *v_cache, const int *table, const int *cache_lens,
                const float *alpha, void *o, int B, int Hq, int Hkv, int Lplan, int d, int dtype, int mode, int k_win,
                int pi, int M, int seg, int layout, int R, int page_shift, int num_pages, int max_pages,
                size_t cache_bytes, void *workspace, size_t workspace_bytes, void *stream,
                const sa::FusedOpts &fo = sa::FusedOpts{}, bool noalloc = false) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || cache_lens == nullptr || o == nullptr)
    return fail(SA_ERR_INVALID, "null tensor pointer");
  if (layout == sa::kCachePaged && table == nullptr) return fail(SA_ERR_INVALID, "null block table");
  int rc = check_opts(fo, mode);
  if (rc != SA_OK) return rc;
  if (mode == SA_MODE_PI && M > 0 && alpha == nullptr && fo.gate_w == nullptr)
    return fail(SA_ERR_INVALID, "alpha is required for PI mode with M > 0");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(alpha, 4) || !aligned(cache_lens, 4) || !aligned(table, 4))
    return fail(SA_ERR_INVALID, "misaligned tensor");
  if ((long long)Lplan * d >= (1LL << 31) || B > 65535) return fail(SA_ERR_INVALID, "problem too large");
  const size_t need = sparse_attn_decode_workspace_size(B, Hq, Hkv, Lplan, d, dtype, mode, k_win, pi, M, seg);
  if (noalloc) {
    if (need > kNoAllocScratchBytes)
      return fail(SA_ERR_WORKSPACE, "decode partial states exceed the 16 MiB device scratch of the allocation-free "
                                    "decode (B * Hq * (window splits + 1) * (d + 4) * 4 bytes); use sparse_attn_decode");
  } else {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(SA_ERR_WORKSPACE, "workspace missing or smaller than the decode workspace size");
    if (!aligned(workspace, 256)) return fail(SA_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * Hq * d * es;
  const size_t ntab = layout == sa::kCachePaged ? (size_t)B * max_pages * 4 : 0;
  if (overlap(o, nq, q, nq) || overlap(o, nq, k_cache, cache_bytes) || overlap(o, nq, v_cache, cache_bytes) ||
      overlap(o, nq, alpha, alpha ? (size_t)B * Hq * 4 : 0) || overlap(o, nq, cache_lens, (size_t)B * 4) ||
      overlap(o, nq, table, ntab) || overlap(o, nq, workspace, need) ||
      overlap(workspace, need, q, nq) || overlap(workspace, need, k_cache, cache_bytes) ||
      overlap(workspace, need, v_cache, cache_bytes) || overlap(workspace, need, cache_lens, (size_t)B * 4) ||
      overlap(workspace, need, table, ntab) || overlap(workspace, need, alpha, alpha ? (size_t)B * Hq * 4 : 0))
    return fail(SA_ERR_INVALID, "output or workspace overlaps another tensor");
  sa::DecodeArgs da;
  da.q = q; da.kc = k_cache; da.vc = v_cache; da.lens = cache_lens; da.alpha = alpha; da.o = o;
  da.ws = (float *)workspace;
  da.B = B; da.Hq = Hq; da.Hkv = Hkv; da.Lmax = Lplan; da.d = d; da.dtype = dtype;
  da.mode = mode; da.k_win = k_win; da.pi = pi; da.M = M; da.seg = seg;
  decode_plan(Lplan, mode, k_win, pi, seg, &da.n_wsplit, &da.chunk, &da.m_min);
  da.nsplit = da.n_wsplit + 1;
  da.layout = layout; da.R = R; da.page_shift = page_shift; da.num_pages = num_pages; da.max_pages = max_pages;
  da.table = table;
  da.opt = fo;
  if (fo.out_gate != nullptr && overlap(o, nq, fo.out_gate, nq)) return fail(SA_ERR_INVALID, "output overlaps out_gate");
  if (noalloc) {   // every argument checked: now the library's device scratch
    rc = scratch_for_current_device(&workspace);
    if (rc != SA_OK) return rc;
    da.ws = (float *)workspace;
  }
  hipError_t e = sa::launch_decode(da, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
  return SA_OK;
}

int decode_head_checks(int B, int Hq, int Hkv, int L, int d, int dtype, int mode, int k_win, int pi, int M, int seg) {
  int rc = check_shape(dtype, d);
  if (rc != SA_OK) return rc;
  if (mode == SA_MODE_WINDOW_BIDIR || mode == SA_MODE_ECP_FULL)
    return fail(SA_ERR_UNSUPPORTED, "a decoded token has no later keys: non-causal masks are prefill-only");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0) return fail(SA_ERR_INVALID, "B, Hq, Hkv and the cache length must be >= 1");
  if (Hq % Hkv != 0) return fail(SA_ERR_INVALID, "Hq must be a multiple of Hkv");
  return check_mode(mode, k_win, pi, M, seg);
}

// Rows a ring must keep: every key of the query at the newest position.
long long ring_span(int mode, int k_win, int pi, int M, int seg) {
  if (mode == SA_MODE_ECP) return 2LL * seg;
  if (mode == SA_MODE_SSPLIT) return seg;
  long long span = (long long)k_win + 1;
  if (mode == SA_MODE_PI && M > 0 && (long long)M * pi + 1 > span) span = (long long)M * pi + 1;
  return span;
}

int page_shift_of(int page_size) {
  if (page_size < 8 || page_size > 4096 || (page_size & (page_size - 1)) != 0) return -1;
  int sh = 0;
  while ((1 << sh) < page_size) ++sh;
  return sh;
}

}  // namespace

int sparse_attn_decode(const void *q, const void *k_cache, const void *v_cache, const int *cache_lens,
                       const float *alpha, void *o, int B, int Hq, int Hkv, int Lmax, int d, int dtype, int mode,
                       int k_win, int pi, int M, int seg, void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  int rc = decode_head_checks(B, Hq, Hkv, Lmax, d, dtype, mode, k_win, pi, M, seg);
  if (rc != SA_OK) return rc;
  if ((long long)B * Hkv * Lmax >= (1LL << 31)) return fail(SA_ERR_INVALID, "problem too large");
  const size_t nc = (size_t)B * Hkv * Lmax * d * elem_size(dtype);
  return decode_impl(q, k_cache, v_cache, nullptr, cache_lens, alpha, o, B, Hq, Hkv, Lmax, d, dtype, mode, k_win, pi,
                     M, seg, sa::kCacheContig, 0, 0, 0, 0, nc, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Device scratch of the allocation-free decode: the split partial states live
// in this file-scope array (one copy per GPU the library runs on, held until
// the process ends).  Host code never passes the array's name to a kernel:
// that name is a host-side stand-in, not a device address.  The address of
// each device's copy is looked up once, with that device current, and kept.
__device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch copy (SA_OK), or an error
// code with the error text set.
int scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
    if (ptr == nullptr) return fail(SA_ERR_HIP, "scratch symbol has no device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

}  // namespace

extern "C" {

size_t sparse_attn_decode_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

int sparse_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int *cache_lens,
                               const float *alpha, void *o, int B, int Hq, int Hkv, int Lmax, int d, int dtype,
                               int mode, int k_win, int pi, int M, int seg, void *stream) {
  g_err[0] = 0;
  int rc = decode_head_checks(B, Hq, Hkv, Lmax, d, dtype, mode, k_win, pi, M, seg);
  if (rc != SA_OK) return rc;
  if ((long long)B * Hkv * Lmax >= (1LL << 31)) return fail(SA_ERR_INVALID, "problem too large");
  const size_t nc = (size_t)B * Hkv * Lmax * d * elem_size(dtype);
  return decode_impl(q, k_cache, v_cache, nullptr, cache_lens, alpha, o, B, Hq, Hkv, Lmax, d, dtype, mode, k_win, pi,
                     M, seg, sa::kCacheContig, 0, 0, 0, 0, nc, nullptr, 0, stream, sa::FusedOpts{}, true);
}

int sparse_attn_decode_ex(const void *q, const void *k_cache, const void *v_cache, const int *cache_lens,
                          const float *alpha, void *o, int B, int Hq, int Hkv, int Lmax, int d, int dtype, int mode,
                          int k_win, int pi, int M, int seg, const sa_options *opt, void *workspace,
                          size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  int rc = decode_head_checks(B, Hq, Hkv, Lmax, d, dtype, mode, k_win, pi, M, seg);
  if (rc != SA_OK) return rc;
  if (dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "decode options take bf16 I/O");
  if ((long long)B * Hkv * Lmax >= (1LL << 31)) return fail(SA_ERR_INVALID, "problem too large");
  const size_t nc = (size_t)B * Hkv * Lmax * d * 2;
  return decode_impl(q, k_cache, v_cache, nullptr, cache_lens, alpha, o, B, Hq, Hkv, Lmax, d, dtype, mode, k_win, pi,
                     M, seg, sa::kCacheContig, 0, 0, 0, 0, nc, workspace, workspace_bytes, stream,
                     fused_opts(opt, Hq));
}

size_t sparse_attn_decode_ring_workspace_size(int B, int Hq, int Hkv, int R, int d, int dtype, int mode, int k_win,
                                              int pi, int M, int seg) {
  if (dtype != SA_DTYPE_BF16 || check_mode(mode, k_win, pi, M, seg) != SA_OK ||
      R < ring_span(mode, k_win, pi, M, seg))
    return 0;
  return sparse_attn_decode_workspace_size(B, Hq, Hkv, R, d, dtype, mode, k_win, pi, M, seg);
}

int sparse_attn_decode_ring(const void *q, const void *k_ring, const void *v_ring, const int *cache_lens,
                            const float *alpha, void *o, int B, int Hq, int Hkv, int R, int d, int dtype, int mode,
                            int k_win, int pi, int M, int seg, void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  int rc = decode_head_checks(B, Hq, Hkv, R, d, dtype, mode, k_win, pi, M, seg);
  if (rc != SA_OK) return rc;
  if (dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "ring caches take bf16 I/O");
  if (R < ring_span(mode, k_win, pi, M, seg))
    return fail(SA_ERR_INVALID, "ring smaller than the key span (k_win + 1, M*pi + 1 or 2*seg)");
  if ((long long)B * Hkv * R >= (1LL << 31)) return fail(SA_ERR_INVALID, "problem too large");
  const size_t nc = (size_t)B * Hkv * R * d * 2;
  return decode_impl(q, k_ring, v_ring, nullptr, cache_lens, alpha, o, B, Hq, Hkv, R, d, dtype, mode, k_win, pi, M,
                     seg, sa::kCacheRing, R, 0, 0, 0, nc, workspace, workspace_bytes, stream);
}

size_t sparse_attn_decode_paged_workspace_size(int B, int Hq, int Hkv, int page_size, int max_pages, int d, int dtype,
                                               int mode, int k_win, int pi, int M, int seg) {
  const int sh = page_shift_of(page_size);
  if (dtype != SA_DTYPE_BF16 || sh < 0 || max_pages <= 0 || (long long)max_pages * page_size >= (1LL << 31) ||
      (mode == SA_MODE_PI && M > 63))
    return 0;
  return sparse_attn_decode_workspace_size(B, Hq, Hkv, max_pages * page_size, d, dtype, mode, k_win, pi, M, seg);
}

int sparse_attn_decode_paged(const void *q, const void *k_pages, const void *v_pages, const int *block_table,
                             const int *cache_lens, const float *alpha, void *o, int B, int Hq, int Hkv,
                             int num_pages, int page_size, int max_pages, int d, int dtype, int mode, int k_win,
                             int pi, int M, int seg, void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  const int sh = page_shift_of(page_size);
  if (sh < 0) return fail(SA_ERR_INVALID, "page_size must be a power of two in [8, 4096]");
  if (max_pages <= 0 || num_pages <= 0) return fail(SA_ERR_INVALID, "num_pages and max_pages must be >= 1");
  if ((long long)max_pages * page_size >= (1LL << 31)) return fail(SA_ERR_INVALID, "problem too large");
  int rc = decode_head_checks(B, Hq, Hkv, max_pages * page_size, d, dtype, mode, k_win, pi, M, seg);
  if (rc != SA_OK) return rc;
  if (dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "paged caches take bf16 I/O");
  if (mode == SA_MODE_PI && M > 63) return fail(SA_ERR_UNSUPPORTED, "paged caches take M <= 63");
  if ((long long)num_pages * Hkv * page_size >= (1LL << 31)) return fail(SA_ERR_INVALID, "page pool too large");
  const size_t nc = (size_t)num_pages * Hkv * page_size * d * 2;
  return decode_impl(q, k_pages, v_pages, block_table, cache_lens, alpha, o, B, Hq, Hkv, max_pages * page_size, d,
                     dtype, mode, k_win, pi, M, seg, sa::kCachePaged, 0, sh, num_pages, max_pages, nc, workspace,
                     workspace_bytes, stream);
}

size_t sparse_attn_bwd_ex_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype, int mode, int k_win,
                                         int pi, int M, int seg, const sa_options *opt) {
  const size_t base = sparse_attn_bwd_workspace_size(B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg);
  if (base == 0) return 0;
  const bool gated = opt != nullptr && opt->out_gate != nullptr;
  return base + (gated ? round_up((size_t)B * Hq * N * d * 2, 256) : 0);
}

size_t sparse_attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype, int mode, int k_win,
                                      int pi, int M, int seg) {
  if (dtype != SA_DTYPE_BF16 || check_shape(dtype, d) != SA_OK || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 ||
      Hq % Hkv != 0 || check_mode(mode, k_win, pi, M, seg) != SA_OK)
    return 0;
  return bwd_layout(B, Hq, N).total;
}

int sparse_attn_bwd(const void *q, const void *k, const void *v, const float *alpha, const void *o, const float *lse,
                    const void *dO, void *dq, void *dk, void *dv, float *dalpha, int B, int Hq, int Hkv, int N, int d,
                    int dtype, int mode, int k_win, int pi, int M, int seg, void *workspace, size_t workspace_bytes,
                    void *stream) {
  return sparse_attn_bwd_ex(q, k, v, alpha, o, lse, dO, dq, dk, dv, dalpha, B, Hq, Hkv, N, d, dtype, mode, k_win, pi,
                            M, seg, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int sparse_attn_bwd_ex(const void *q, const void *k, const void *v, const float *alpha, const void *o,
                       const float *lse, const void *dO, void *dq, void *dk, void *dv, float *dalpha, int B, int Hq,
                       int Hkv, int N, int d, int dtype, int mode, int k_win, int pi, int M, int seg,
                       const sa_options *opt, void *dgate, void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  const sa::FusedOpts fo = fused_opts(opt, Hq);
  int rc = check_shape(dtype, d);
  if (rc != SA_OK) return rc;
  if (dtype != SA_DTYPE_BF16) return fail(SA_ERR_UNSUPPORTED, "the backward pass supports bf16 I/O only");
  rc = check_opts(fo, mode);
  if (rc != SA_OK) return rc;
  if (fo.cosine || fo.gate_w != nullptr)
    return fail(SA_ERR_UNSUPPORTED, "the backward pass takes the score scale and the output gate, not cosine scores or the query-driven gate");
  const bool out_gated = fo.out_gate != nullptr;
  if (out_gated && (dgate == nullptr || !aligned(dgate, 16)))
    return fail(SA_ERR_INVALID, "an output gate needs a 16-byte aligned dgate");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return fail(SA_ERR_INVALID, "B, Hq, Hkv and N must be >= 1");
  if (Hq % Hkv != 0) return fail(SA_ERR_INVALID, "Hq must be a multiple of Hkv");
  rc = check_mode(mode, k_win, pi, M, seg);
  if (rc != SA_OK) return rc;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr || dO == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return fail(SA_ERR_INVALID, "null tensor pointer");
  const bool gated = mode == SA_MODE_PI && M > 0;
  if (gated && alpha == nullptr) return fail(SA_ERR_INVALID, "alpha is required for PI mode with M > 0");
  if (mode == SA_MODE_PI && alpha != nullptr && dalpha == nullptr)
    return fail(SA_ERR_INVALID, "dalpha is required when alpha is given (PI mode)");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(alpha, 4) ||
      !aligned(dalpha, 4))
    return fail(SA_ERR_INVALID, "misaligned tensor");
  const long long rows = (long long)B * Hq * N;
  if (rows >= (1LL << 31) || (long long)N * d >= (1LL << 31)) return fail(SA_ERR_INVALID, "problem too large");
  const bool skips = has_skips(mode, k_win, pi, M, N);
  const BwdLayout L = bwd_layout(B, Hq, N);
  const size_t nq = (size_t)rows * d * 2, nkv = (size_t)B * Hkv * N * d * 2, nr = (size_t)rows * 4;
  const size_t total = L.total + (out_gated ? round_up(nq, 256) : 0);
  if (workspace == nullptr || workspace_bytes < total)
    return fail(SA_ERR_WORKSPACE, "workspace missing or smaller than the backward workspace size");
  if (!aligned(workspace, 256)) return fail(SA_ERR_INVALID, "workspace must be 256-byte aligned");
  const void *ins[] = {q, k, v, o, dO, lse, alpha, workspace, fo.out_gate};
  const size_t insz[] = {nq, nkv, nkv, nq, nq, nr, alpha ? nr : 0, total, out_gated ? nq : 0};
  void *outs[] = {dq, dk, dv, dalpha, out_gated ? dgate : nullptr};
  const size_t outsz[] = {nq, nkv, nkv, dalpha ? nr : 0, out_gated ? nq : 0};
  for (int a = 0; a < 5; ++a) {
    for (int bb = 0; bb < 9; ++bb)
      if (overlap(outs[a], outsz[a], ins[bb], insz[bb])) return fail(SA_ERR_INVALID, "a gradient overlaps an input or the workspace");
    for (int bb = 0; bb < 5; ++bb)
      if (bb != a && overlap(outs[a], outsz[a], outs[bb], outsz[bb])) return fail(SA_ERR_INVALID, "gradients overlap");
  }
  sa::BwdArgs ba;
  ba.q = q; ba.k = k; ba.v = v; ba.o = o; ba.dO = dO; ba.alpha = mode == SA_MODE_PI ? alpha : nullptr; ba.lse = lse;
  ba.dq = dq; ba.dk = dk; ba.dv = dv; ba.dalpha = mode == SA_MODE_PI && alpha != nullptr ? dalpha : nullptr;
  char *w = (char *)workspace;
  ba.Dv = (float *)(w + L.dv_off);
  ba.cv = (float *)(w + L.cv_off);
  ba.skips = skips ? 1 : 0;
  ba.B = B; ba.Hq = Hq; ba.Hkv = Hkv; ba.N = N; ba.d = d;
  ba.mode = mode; ba.k_win = k_win; ba.pi = pi; ba.M = M; ba.seg = seg;
  ba.m_min = skips ? (int)skip_m_min(k_win, pi) : 1;
  ba.score_scale = fo.score_scale;
  ba.out_gate = fo.out_gate;
  ba.dgate = out_gated ? dgate : nullptr;
  ba.dO_gated = out_gated ? (void *)(w + L.total) : nullptr;
  hipError_t e = sa::launch_bwd(ba, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SA_ERR_HIP, hipGetErrorString(e));
  return SA_OK;
}

const char *sparse_attn_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_HIP: return "HIP error";
    case SA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char *sparse_attn_last_error(void) { return g_err; }

int sparse_attn_version(void) { return 101; }

}  // extern "C"
