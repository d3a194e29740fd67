/*
 * sparse_attn.h -- C ABI of the causal structured-sparse attention library
 * for AMD Instinct MI355X (gfx950).  Library: libsparse_attn.so.
 *
 * Operation.  For every query position i the library takes ONE softmax over
 * an explicit key set and returns the weighted sum of the value rows:
 *
 *   o_i = sum_{j in K(i)} softmax_j( <q_i, k_j> / sqrt(d) + prior(i, j) ) v_j
 *
 * with the key set K(i) fixed by the mode:
 *
 *   SA_MODE_PI      pi-Attention ("pi-Attention: Periodic Sparse Transformers
 *                   for Efficient Long-Context Modeling", section 2, items
 *                   1-3): the causal window [max(0, i-k_win), i] united with
 *                   the periodic skip keys i - m*pi, m = 1..M, i - m*pi >= 0.
 *                   A skip position inside the window counts once, as a local
 *                   key.  Gate alpha (per query token and query head) enters
 *                   as a log-prior: log(alpha) on local scores, log(1-alpha)
 *                   on skip scores.  alpha must lie in (0, 1]; alpha = 1
 *                   removes the skip keys.
 *   SA_MODE_WINDOW  window-only sparse attention ("LT2: Linear-Time Looped
 *                   Transformers", section 2.1): the causal window alone, no
 *                   prior (the same as SA_MODE_PI with M = 0).
 *   SA_MODE_ECP     paired-half-segment attention ("Efficient Context
 *                   Propagating Perceiver Architectures for Auto-Regressive
 *                   Language Modeling", section 2, PAR block): a query in
 *                   half-segment c = floor(i / seg) attends the keys of
 *                   half-segments c-1 and c, causally: [max(0,(c-1)*seg), i].
 *   Further masks (no prior; prefill forward and backward, and decode where
 *   the mask is causal):
 *   SA_MODE_WINDOW_BIDIR  the two-sided window [max(0,i-k_win), min(N-1,i+k_win)],
 *                   the local window exactly as the pi-Attention page states
 *                   it (encoder use; not a decode mode).
 *   SA_MODE_SSPLIT  s-Split segments (ECP page, section 2): the sequence cut
 *                   into disjoint segments of seg positions, causal inside:
 *                   [floor(i/seg)*seg, i].
 *   SA_MODE_ECP_FULL  the PAR block without the causal restriction: a query in
 *                   half-segment c attends all of half-segments c-1 and c,
 *                   [max(0,(c-1)*seg), min(N-1,(c+1)*seg-1)] (not a decode mode).
 *
 * Grouped-query attention (the attention branch of the hybrid GSS-Transformer
 * page, methodology item 1): query head h reads key/value head
 * h / (Hq / Hkv).
 *
 * Conventions shared by every entry point.
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous.
 *     q/k/v/o/caches must be 16-byte aligned, alpha/lens 4-byte aligned.
 *   - dtype SA_DTYPE_BF16: q, k, v, o (and caches) hold bfloat16; scores,
 *     softmax and accumulation run in fp32; o is rounded to nearest even.
 *     dtype SA_DTYPE_F32: everything is fp32.  alpha is fp32 in both.
 *   - Head dimension d must be 64 or 128 (else SA_ERR_UNSUPPORTED).
 *   - The caller owns every buffer, including the workspace.  The library
 *     allocates no device memory and never synchronises.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL =
 *     the default stream).  The return value only reports argument and launch
 *     errors; a fault inside a kernel surfaces at the caller's next
 *     synchronisation.
 *   - Argument errors are detected on the host before any HIP call, and then
 *     nothing is launched.  sparse_attn_last_error() gives the detail (per
 *     thread).  NaN/Inf in the data propagate without checks; alpha outside
 *     (0, 1] gives undefined (non-finite) outputs for the affected rows.
 *   - Parameters a mode does not use are ignored (PI: k_win, pi, M, alpha;
 *     WINDOW: k_win; ECP: seg).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SA_OK 0
#define SA_ERR_INVALID (-1)     /* bad pointer, size, parameter, alignment or aliasing */
#define SA_ERR_UNSUPPORTED (-2) /* head dim or dtype outside what is built */
#define SA_ERR_HIP (-3)         /* a HIP launch or query failed */
#define SA_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required */

/* Modes. */
#define SA_MODE_PI 0
#define SA_MODE_WINDOW 1
#define SA_MODE_ECP 2
#define SA_MODE_WINDOW_BIDIR 3
#define SA_MODE_SSPLIT 4
#define SA_MODE_ECP_FULL 5

/* I/O element types. */
#define SA_DTYPE_F32 0
#define SA_DTYPE_BF16 1

/*
 * Bytes of device workspace sparse_attn_fwd needs for these arguments (0 when
 * none is needed: WINDOW, ECP, and PI when no query has a skip key).  Returns
 * 0 as well for arguments sparse_attn_fwd would reject.
 */
size_t sparse_attn_fwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype,
                                      int mode, int k_win, int pi, int M, int seg);

/*
 * Prefill forward.
 *   q     [B, Hq,  N, d]   k, v [B, Hkv, N, d]   o [B, Hq, N, d] (dtype)
 *   alpha [B, Hq, N] fp32, required when mode == SA_MODE_PI and M > 0 (may be
 *         NULL otherwise).
 *   Requires B, Hq, Hkv, N >= 1, Hq % Hkv == 0, k_win >= 0; for PI with M > 0
 *   pi >= 1; M >= 0; for ECP seg >= 1.  o must not overlap q, k, v, alpha or
 *   the workspace.
 *   workspace: device buffer of at least sparse_attn_fwd_workspace_size(...)
 *   bytes, 256-byte aligned (NULL allowed when that size is 0).  Its contents
 *   are scratch; it must not be shared by calls that may run concurrently.
 * Returns SA_OK or an error code.
 */
int sparse_attn_fwd(const void *q, const void *k, const void *v, const float *alpha, void *o,
                    int B, int Hq, int Hkv, int N, int d, int dtype,
                    int mode, int k_win, int pi, int M, int seg,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training forward: sparse_attn_fwd (same arguments, workspace and errors)
 * that also writes the log-sum-exp of every row's scores,
 *   lse[b, h, i] = log sum_{j in K(i)} exp(<q_i, k_j>/sqrt(d) + prior(i, j)),
 * fp32 [B, Hq, N], natural log; the backward pass reads it.  lse must not be
 * NULL nor overlap another tensor.
 */
int sparse_attn_fwd_lse(const void *q, const void *k, const void *v, const float *alpha, void *o,
                        float *lse, int B, int Hq, int Hkv, int N, int d, int dtype,
                        int mode, int k_win, int pi, int M, int seg,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace sparse_attn_bwd needs (0 for arguments it would
 * reject, including dtype != SA_DTYPE_BF16).
 */
size_t sparse_attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype,
                                      int mode, int k_win, int pi, int M, int seg);

/*
 * Backward pass: gradients of a scalar loss L given dO = dL/dO, through the
 * forward's single softmax over each key set with the gate as a log-prior
 * (pi-Attention section 2 item 3 for the gate):
 *   dq [B,Hq,N,d], dk and dv [B,Hkv,N,d] (bf16; dk, dv summed over the query
 *   heads of each GQA group), dalpha [B,Hq,N] fp32 (PI mode when alpha is
 *   given; may be NULL otherwise) with
 *   dL/dalpha_i = sum_{j local} dS_ij / alpha_i - sum_{j skip} dS_ij / (1 - alpha_i),
 *   dS_ij = P_ij (<dO_i, v_j> - <dO_i, o_i>) the gradient of score (i, j);
 *   as sum_j dS_ij = 0, it is computed as -sum_{j skip} dS_ij / (alpha_i (1 - alpha_i))
 *   (0 on rows without skip keys, finite at alpha_i = 1).
 *   o, lse: the outputs of sparse_attn_fwd_lse for the same q, k, v, alpha.
 *   bf16 I/O only (SA_ERR_UNSUPPORTED otherwise); d in {64, 128}.  No output
 *   may overlap an input, another output or the workspace.
 *   workspace: >= sparse_attn_bwd_workspace_size(...) bytes, 256-byte
 *   aligned; scratch, not to be shared by concurrent calls.
 * Returns SA_OK or an error code.
 */
int sparse_attn_bwd(const void *q, const void *k, const void *v, const float *alpha,
                    const void *o, const float *lse, const void *dO,
                    void *dq, void *dk, void *dv, float *dalpha,
                    int B, int Hq, int Hkv, int N, int d, int dtype,
                    int mode, int k_win, int pi, int M, int seg,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace sparse_attn_decode needs (never 0 for valid
 * arguments; 0 for arguments sparse_attn_decode would reject).
 */
size_t sparse_attn_decode_workspace_size(int B, int Hq, int Hkv, int Lmax, int d, int dtype,
                                         int mode, int k_win, int pi, int M, int seg);

/*
 * Single-token decode over a KV cache (autoregressive decoding, where the
 * pi-Attention page restricts every key to earlier positions).  For sequence
 * b the new token's query sits at position i = cache_lens[b] - 1 and the
 * cache already holds that token's key and value; the query attends K(i) of
 * the mode, read from rows [b, h / (Hq/Hkv), j, :] of the caches.
 *   q          [B, Hq, d]               o [B, Hq, d] (dtype)
 *   k_cache, v_cache [B, Hkv, Lmax, d]  (the prefill k/v layout with N = Lmax)
 *   cache_lens [B] int32, DEVICE memory; each value must lie in [1, Lmax].
 *              A row whose length lies outside that range reads nothing and
 *              gets NaN outputs.
 *   alpha      [B, Hq] fp32 (PI with M > 0; NULL allowed otherwise).
 *   workspace  >= sparse_attn_decode_workspace_size(...) bytes, 256-byte
 *              aligned; scratch, not to be shared by concurrent calls.
 * Returns SA_OK or an error code.
 */
int sparse_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                       const int *cache_lens, const float *alpha, void *o,
                       int B, int Hq, int Hkv, int Lmax, int d, int dtype,
                       int mode, int k_win, int pi, int M, int seg,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same operation, arguments and results as
 * sparse_attn_decode over a contiguous cache, without the workspace
 * arguments: the split partial states go to a device scratch array that the
 * library holds for each GPU it runs on (16 MiB, kept until the process
 * ends; its address is looked up on the first call on each device, with that
 * device current).  The call allocates nothing.
 *   Limit: sparse_attn_decode_workspace_size(...) of the same arguments must
 *   not exceed sparse_attn_decode_noalloc_max_workspace() (16 MiB), else
 *   SA_ERR_WORKSPACE and nothing is launched.
 *   Every call on one GPU uses that GPU's one scratch array: calls that
 *   overlap in time on the same GPU (different streams or threads without
 *   ordering between them) race and give undefined results.  Calls ordered
 *   on one stream are safe.  Nothing in the scratch needs clearing between
 *   calls (every partial state a call reads was written by that call).
 */
size_t sparse_attn_decode_noalloc_max_workspace(void);
int sparse_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                               const int *cache_lens, const float *alpha, void *o,
                               int B, int Hq, int Hkv, int Lmax, int d, int dtype,
                               int mode, int k_win, int pi, int M, int seg, void *stream);

/*
 * Serving-cache layouts for the same decode (bf16 I/O only; fp32 returns
 * SA_ERR_UNSUPPORTED).  Semantics, q, alpha, o, cache_lens and workspace as
 * sparse_attn_decode; only where a position's key/value row lives differs.
 *
 * Ring cache: k_ring, v_ring [B, Hkv, R, d]; position p of sequence b lives in
 * slot p mod R, so a stream of any length keeps only its last R tokens.  The
 * keys of the query at position len - 1 must all still be resident: R must be
 * at least the key span, k_win + 1 and (PI with M > 0) M*pi + 1, or 2*seg for
 * ECP (else SA_ERR_INVALID).  cache_lens[b] >= 1 counts the tokens written so
 * far (no upper bound); a length < 1 gives NaN outputs.
 */
size_t sparse_attn_decode_ring_workspace_size(int B, int Hq, int Hkv, int R, int d, int dtype,
                                              int mode, int k_win, int pi, int M, int seg);
int sparse_attn_decode_ring(const void *q, const void *k_ring, const void *v_ring,
                            const int *cache_lens, const float *alpha, void *o,
                            int B, int Hq, int Hkv, int R, int d, int dtype,
                            int mode, int k_win, int pi, int M, int seg,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Paged cache: a pool of num_pages pages, k_pages, v_pages
 * [num_pages, Hkv, page_size, d] (a page holds page_size consecutive positions
 * of one sequence for every KV head), and block_table int32 [B, max_pages] in
 * DEVICE memory: logical page j = p / page_size of sequence b is physical page
 * block_table[b, j].  page_size is a power of two in [8, 4096]; PI mode takes
 * M <= 63 (else SA_ERR_UNSUPPORTED).  cache_lens[b] must lie in
 * [1, max_pages * page_size]; a length outside that range, or a table entry
 * the query needs that lies outside [0, num_pages), gives NaN outputs for that
 * sequence and reads no cache row.
 */
size_t sparse_attn_decode_paged_workspace_size(int B, int Hq, int Hkv, int page_size, int max_pages,
                                               int d, int dtype, int mode, int k_win, int pi, int M,
                                               int seg);
int sparse_attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                             const int *block_table, const int *cache_lens, const float *alpha,
                             void *o, int B, int Hq, int Hkv, int num_pages, int page_size,
                             int max_pages, int d, int dtype, int mode, int k_win, int pi, int M,
                             int seg, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Fused gate and epilogue options (the *_ex entry points).  A NULL options
 * pointer, or a zero-initialised struct, means the plain operation.
 *   score_scale  > 0: scores use this scale instead of 1/sqrt(d).
 *   cosine       nonzero: scaled cosine scores, score_scale * cos(q_i, k_j)
 *                (the attention branch of the hybrid GSS-Transformer page,
 *                methodology item 1); q and k rows must be nonzero.  The
 *                forward keeps an L2-normalised copy of k in the workspace.
 *   gate_w, gate_b, gate_hidden, gate_w2, gate_b2
 *                PI mode: the gate is computed in-kernel from the query by a
 *                light per-token, per-head network (pi-Attention section 2
 *                item 3: an MLP produces alpha), and the alpha argument is
 *                ignored.  The query row is the network's input.
 *                gate_hidden = H in [1, 32]: two layers with a ReLU hidden
 *                layer of width H,
 *                  alpha_i = sigmoid( sum_u gate_w2[h][u] *
 *                            relu(<gate_w[h][u], q_i> + gate_b[h][u]) + gate_b2[h] ),
 *                  gate_w fp32 [Hq, H, d], gate_b [Hq, H], gate_w2 [Hq, H],
 *                  gate_b2 [Hq].  The first layer runs on the matrix cores
 *                  with each fp32 weight split into two bf16 parts.
 *                gate_hidden = 0: one linear layer,
 *                  alpha_i = sigmoid(<gate_w[h], q_i> + gate_b[h]),
 *                  gate_w fp32 [Hq, d], gate_b [Hq]; gate_w2, gate_b2 NULL.
 *                Device memory; gate_w 16-byte aligned, the others 4-byte.
 *                gate_w and gate_b go together; SA_ERR_INVALID for a missing
 *                second layer, H outside [0, 32], or the gate outside PI mode.
 *   out_gate     output gate of the LT2 page (section 3): the result is
 *                o * sigmoid(out_gate), out_gate shaped and typed like o
 *                (decode: [B, Hq, d]), device memory, 16-byte aligned.
 */
typedef struct sa_options {
  float score_scale;
  int cosine;
  const float *gate_w;
  const float *gate_b;
  const void *out_gate;
  int gate_hidden;
  const float *gate_w2;
  const float *gate_b2;
} sa_options;

/*
 * sparse_attn_fwd / sparse_attn_fwd_lse with options (lse may be NULL).
 * Workspace: sparse_attn_fwd_ex_workspace_size (cosine adds B*Hkv*N*d
 * elements for the normalised keys).  Errors as sparse_attn_fwd, plus
 * SA_ERR_INVALID for a bad option (negative or non-finite score_scale, only
 * one of gate_w / gate_b, the gate outside PI mode, misalignment, out_gate
 * overlapping o).
 */
size_t sparse_attn_fwd_ex_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype,
                                         int mode, int k_win, int pi, int M, int seg,
                                         const sa_options *opt);
int sparse_attn_fwd_ex(const void *q, const void *k, const void *v, const float *alpha, void *o,
                       float *lse, int B, int Hq, int Hkv, int N, int d, int dtype,
                       int mode, int k_win, int pi, int M, int seg, const sa_options *opt,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * sparse_attn_decode (contiguous caches) with options; bf16 I/O only
 * (SA_ERR_UNSUPPORTED otherwise).  Workspace as sparse_attn_decode.
 */
int sparse_attn_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                          const int *cache_lens, const float *alpha, void *o,
                          int B, int Hq, int Hkv, int Lmax, int d, int dtype,
                          int mode, int k_win, int pi, int M, int seg, const sa_options *opt,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * sparse_attn_bwd with options: score_scale and out_gate (cosine and the
 * query-driven gate return SA_ERR_UNSUPPORTED).  With out_gate, o is the
 * gated output y = o_attn * sigmoid(g) of sparse_attn_fwd_ex, dO is dL/dy,
 * and dgate [B, Hq, N, d] bf16 receives dL/dg = dO * y * (1 - sigmoid(g));
 * the workspace (sparse_attn_bwd_ex_workspace_size) adds B*Hq*N*d bf16.
 */
size_t sparse_attn_bwd_ex_workspace_size(int B, int Hq, int Hkv, int N, int d, int dtype,
                                         int mode, int k_win, int pi, int M, int seg,
                                         const sa_options *opt);
int sparse_attn_bwd_ex(const void *q, const void *k, const void *v, const float *alpha,
                       const void *o, const float *lse, const void *dO,
                       void *dq, void *dk, void *dv, float *dalpha,
                       int B, int Hq, int Hkv, int N, int d, int dtype,
                       int mode, int k_win, int pi, int M, int seg, const sa_options *opt,
                       void *dgate, void *workspace, size_t workspace_bytes, void *stream);

/* Static text for a status code. */
const char *sparse_attn_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *sparse_attn_last_error(void);

/* Library ABI version (major * 100 + minor). */
int sparse_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
