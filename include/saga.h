/*
 * saga.h - C ABI of the SAGA + Atop-N single-token decode-attention library (gfx950).
 *
 * The operation (paper "More Value per Key: Asymmetric Sparse Attention for Faster
 * LLM Decoding", summary page picx.dev DRD92V):
 *   - eq. (2): A[b,j,i] = (q[b,j,:] . K[b,g(j),i,:]) * scale over the l_kv[b] cached keys,
 *     with only h_k key heads (section "SAGA Architecture");
 *   - section "Methodology > Atop-N Attention": entries are kept by comparing A with a
 *     per-row threshold, the N-th largest logit of the row; the exact threshold is
 *     recomputed once every `refresh_period` decode steps (the pages' n) and reused;
 *   - eq. (7): O[b,j,:] = softmax(A[b,j,S]) V[b,v(j),S,:] over the kept set S, with
 *     h_v >= h_k value heads.
 *   g(j) = floor(j*h_k/h_q), v(j) = floor(j*h_v/h_q) (contiguous head groups).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns all memory;
 *     the library allocates nothing, keeps no pointer after returning, never
 *     synchronises the stream, never prints and never aborts.
 *   - Layouts (row-major, contiguous): q [B,h_q,d]; K [B,h_k,l_max,d]; V [B,h_v,l_max,d_v];
 *     out [B,h_q,d_v]; l_kv [B] int32; tau [B,h_q] float32. d is the query/key head
 *     dimension, d_v the value head dimension (saga_shape.d_v).
 *   - Cache rows read: rows >= max_l_kv are never read, and rows >= l_kv[b] never
 *     contribute to a result. With batch 1 the loads of a call are issued before
 *     l_kv[0] is known, so rows l_kv[0] .. max_l_kv - 1 may be read and discarded
 *     (key rows by the decode calls, key and value rows by the dense calls); they lie
 *     inside the caches, since max_l_kv <= l_max, and whatever they hold (even NaN)
 *     never reaches a result. With batch > 1, rows at or past l_kv[b] are never read,
 *     and the decode calls read value rows only for kept entries.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Results are valid once the stream reaches the call.
 *   - Arguments are checked on the host before anything is launched; on any error
 *     nothing is enqueued and no output is written.
 *   - Device-side values cannot be checked: l_kv[b] must lie in [0, max_l_kv] and the
 *     inputs must be finite. l_kv[b] == 0 yields a zero output row, sel_count 0 and an
 *     unchanged threshold.
 *   - Workspace: `saga_workspace_bytes` bytes of device memory, zero-filled before
 *     its first use (saga_workspace_init does that). Every call leaves the counters it
 *     uses back at zero, so a workspace is reused across calls without clearing.
 *     Calls sharing one workspace must be ordered on one stream; concurrent calls
 *     need separate workspaces.
 */
#ifndef SAGA_H
#define SAGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum saga_status {
  SAGA_OK = 0,
  SAGA_ERR_NULL = 1,        /* a required pointer is NULL */
  SAGA_ERR_SHAPE = 2,       /* inconsistent sizes: heads not divisible, N < 1, period < 1, ... */
  SAGA_ERR_UNSUPPORTED = 3, /* valid but not built: (d, d_v) not built, unknown dtype, too long,
                               too many (sequence, head) rows */
  SAGA_ERR_WORKSPACE = 4,   /* workspace smaller than saga_workspace_bytes() */
  SAGA_ERR_HIP = 5          /* the HIP runtime reported an error at launch */
} saga_status;

typedef enum saga_dtype { SAGA_F32 = 0, SAGA_BF16 = 1 } saga_dtype;

/* Head counts and sizes, named as on the pages (section "Attention Mechanism
 * Formalization": h heads of dimension d; section "SAGA Architecture": h_k, h_v). */
typedef struct saga_shape {
  int32_t batch;      /* B >= 1 sequences, one decode token each; B <= 65535 */
  int32_t h_q;        /* query heads; multiple of h_k and of h_v; h_q <= 65535, B h_q <= 2^24 */
  int32_t h_k;        /* key heads */
  int32_t h_v;        /* value heads */
  int32_t d;          /* head dimension of q and K (d_k): 32, 64 or 128, see d_v */
  int32_t d_v;        /* head dimension of V and out; 0 means d. Built: d_v == d in {64, 128},
                       * and the reduced key dimensions (d, d_v) = (32, 64), and (64, 128)
                       * for bf16 (section "Training from Scratch": a key head dimension
                       * below the value head dimension). The logit scale is 1/sqrt(d). */
  int32_t l_max;      /* cache capacity: row stride (in tokens) of K and V; at most 2^24 */
  int32_t dtype;      /* saga_dtype of q, K and V */
  int32_t out_dtype;  /* saga_dtype of out (bf16 output is rounded to nearest even) */
  float scale;        /* logit scale; 0 selects 1/sqrt(d) as in eq. (2) */
} saga_shape;

/* Status name, e.g. "SAGA_ERR_SHAPE"; a static string, never NULL. */
const char* saga_status_str(int32_t status);

/* Bytes of workspace the calls below need for `s`, top-N size N and contexts up to
 * max_l_kv tokens. 0 if the shape is invalid. Pure host arithmetic. The size never
 * decreases with max_l_kv, so a workspace sized for a context serves every call with
 * a smaller max_l_kv (a growing decode context allocates once). */
size_t saga_workspace_bytes(const saga_shape* s, int32_t N, int32_t max_l_kv);

/* The form of the value gather that saga_decode_attn (and saga_select_gather with
 * saga_split_combine) takes for `s`, top-N size N and max_l_kv: 1 for the late gather
 * (the combining kernel reads the kept value rows), 0 for the early gather (the
 * select kernel does), -1 if the arguments are invalid. saga_decode_attn_paged always
 * takes the early gather. Pure host arithmetic; the results of the step do not depend
 * on the form beyond the rounding of its sums. */
int32_t saga_gather_form(const saga_shape* s, int32_t N, int32_t max_l_kv);

/* Enqueue a zero fill of `bytes` bytes of `workspace` (first-use initialisation). */
saga_status saga_workspace_init(void* workspace, size_t bytes, void* stream);

/* One SAGA + Atop-N decode step (eq. (2), the Atop-N threshold rule, eq. (7)).
 *   max_l_kv (host): upper bound of l_kv[], sizes the launch grid.
 *   N: top-N size (>= 1). refresh_period (>= 1) and step (host) choose the exact
 *     threshold refresh: when step % refresh_period == 0, tau[b,j] is recomputed as the
 *     N-th largest fp32 logit of its row (-inf when N >= l_kv[b]) before selecting;
 *     otherwise the tau passed in is used as is.
 *   tau [B,h_q] in/out: the per-(sequence, query head) threshold state. At a refresh
 *     step the value passed in only guesses where the new threshold lies (a refresh whose
 *     threshold moved little since the last one takes the faster path); the results
 *     never depend on it.
 *   Kept set S[b,j] = { i < l_kv[b] : A[b,j,i] >= tau[b,j] } (ties kept). If a stale
 *     threshold keeps nothing, that row is refreshed exactly at this step.
 *   out [B,h_q,d_v] (out_dtype): eq. (7) over S.
 *   sel_count [B,h_q] (optional, may be NULL): |S[b,j]|.
 *   sel_idx [B,h_q,sel_cap] (optional): the first min(|S|, sel_cap) kept indices,
 *     in no particular order; entries past that are left untouched.
 *   flags [B,h_q] (optional): bit 0 = the threshold was refreshed at this step,
 *     bit 1 = the refresh was forced by an empty stale selection. */
saga_status saga_decode_attn(const saga_shape* s, const void* q, const void* k, const void* v,
                             const int32_t* l_kv, int32_t max_l_kv, int32_t N,
                             int32_t refresh_period, int64_t step, float* tau, void* out,
                             int32_t* sel_count, int32_t* sel_idx, int32_t sel_cap,
                             int32_t* flags, void* workspace, size_t workspace_bytes,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): saga_decode_attn with its workspace
 * in a scratch array inside the library instead of a caller's buffer. Arguments,
 * results and errors are those of saga_decode_attn, plus:
 *   - Scratch: SAGA_NOALLOC_SCRATCH_BYTES of device memory per GPU, set up by the HIP
 *     runtime when the library's code is loaded on that GPU and held until the process
 *     ends. The call uses the copy of the current device (hipGetDevice); `stream` must
 *     belong to that device. The first call on a device looks up the copy's address
 *     (SAGA_ERR_HIP if that fails); nothing is ever allocated or freed (no hipMalloc,
 *     no hipFree, no allocating library call).
 *   - SAGA_ERR_WORKSPACE when the step needs more than the scratch holds, i.e. when
 *     saga_workspace_bytes(s, N, max_l_kv) > SAGA_NOALLOC_SCRATCH_BYTES (one sequence
 *     of 128K tokens with 12 query heads of 128 needs about 25 MiB; a batch of 16
 *     such sequences does not fit). Checked before anything is enqueued.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last call's
 *     contents: calls that overlap on one GPU (concurrent streams, or host threads
 *     enqueueing at once) race and give undefined results; order them on one stream.
 *     A refresh step first clears the scratch's threshold counters with a fill kernel
 *     (one extra launch, no memset node), so no earlier contents are relied on. */
#define SAGA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
saga_status saga_decode_attn_noalloc(const saga_shape* s, const void* q, const void* k, const void* v,
                                     const int32_t* l_kv, int32_t max_l_kv, int32_t N,
                                     int32_t refresh_period, int64_t step, float* tau, void* out,
                                     int32_t* sel_count, int32_t* sel_idx, int32_t sel_cap,
                                     int32_t* flags, void* stream);

/* The exact threshold alone (section "Methodology > Atop-N Attention", refresh step):
 * tau[b,j] = N-th largest fp32 logit of row (b,j), counting repeats; -inf when
 * N >= l_kv[b]; unchanged when l_kv[b] == 0. The value tau holds on entry only guesses
 * where the new one lies (as for saga_decode_attn); any value, NaN included, gives the
 * same result. */
saga_status saga_refresh_threshold(const saga_shape* s, const void* q, const void* k,
                                   const int32_t* l_kv, int32_t max_l_kv, int32_t N,
                                   float* tau, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Dense attention, eq. (2)-(4) over every cached key and value, with query head j
 * reading key head g(j) and value head v(j). With h_k == h_v this is grouped-query
 * attention, the baseline the pages compare against (Figure 2); with h_k < h_v it is
 * SAGA with full attention (section "SAGA Architecture" without Atop-N selection).
 * SAGA_ERR_UNSUPPORTED unless h_k divides h_v and h_q / h_v <= 16. */
saga_status saga_dense_gqa_attn(const saga_shape* s, const void* q, const void* k,
                                const void* v, const int32_t* l_kv, int32_t max_l_kv,
                                void* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The two stages of a non-refresh decode step, callable separately on one stream
 * with one workspace: saga_qk_select followed by saga_sparse_gather computes the step
 * of saga_decode_attn with step % refresh_period != 0 (the same kept sets, counts and
 * flags; outputs equal up to the rounding of sums taken in another order).
 * saga_qk_select: scores every cached key of the h_k key heads (eq. (2)) and keeps,
 *   per query head, the entries >= tau into the workspace (Atop-N comparison step).
 * saga_sparse_gather: softmax over the kept entries and the gather of their value
 *   rows (eq. (7)); outputs as in saga_decode_attn (flags bit 0 is never set here).
 *   q, k, N and tau are needed for the forced refresh of a row that kept nothing. */
saga_status saga_qk_select(const saga_shape* s, const void* q, const void* k,
                           const int32_t* l_kv, int32_t max_l_kv, const float* tau,
                           void* workspace, size_t workspace_bytes, void* stream);
saga_status saga_sparse_gather(const saga_shape* s, const void* q, const void* k,
                               const void* v, const int32_t* l_kv, int32_t max_l_kv,
                               int32_t N, float* tau, void* out, int32_t* sel_count,
                               int32_t* sel_idx, int32_t sel_cap, int32_t* flags,
                               void* workspace, size_t workspace_bytes, void* stream);

/* The two kernels of a step that reuses the threshold, callable separately on one
 * stream with one workspace (saga_decode_attn with step % refresh_period != 0 is
 * exactly saga_select_gather followed by saga_split_combine with the same N). Both
 * take one of two forms, chosen from the shape, N and max_l_kv exactly as
 * saga_decode_attn chooses it (saga_gather_form): contiguous caches with value rows
 * of at least 256 bytes, rows of at most 512 runs of cached keys (the kernel's chunk,
 * 128 to 512 keys), at least 512 runs over all key heads and sequences, and a head
 * expected to keep at most 1 entry per run (at most 2 with 2048 runs or more) take
 * the late value gather; other shapes and selections the early one.
 * saga_select_gather: eq. (2) logits of every cached key and the comparison with tau,
 *   then per chunk and query head, into the workspace:
 *   - early gather: the part of eq. (7) over the chunk's kept entries relative to
 *     their largest logit m_c, sum exp(A_i - m_c) V[i,:] and sum exp(A_i - m_c);
 *   - late gather: the kept (index, logit) pairs, their count and largest logit.
 * saga_split_combine: eq. (7) into out; early gather: the log-sum-exp merge of the
 *   chunk parts (O = sum_c e_c o_c / sum_c e_c z_c, e_c = exp(m_c - max_c m_c)); late
 *   gather: exp(A_i - M) with M the row's largest kept logit, and the gather of the
 *   kept value rows. Outputs as in saga_decode_attn (flags bit 0 is never set here).
 *   q, k, N and tau are needed for the forced refresh of a row that kept nothing. */
saga_status saga_select_gather(const saga_shape* s, const void* q, const void* k,
                               const void* v, const int32_t* l_kv, int32_t max_l_kv,
                               int32_t N, const float* tau, void* workspace,
                               size_t workspace_bytes, void* stream);
saga_status saga_split_combine(const saga_shape* s, const void* q, const void* k,
                               const void* v, const int32_t* l_kv, int32_t max_l_kv,
                               int32_t N, float* tau, void* out, int32_t* sel_count,
                               int32_t* sel_idx, int32_t sel_cap, int32_t* flags,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Paged (non-contiguous) caches for batched decode (the batch-16 setting of the
 * summary page's section "Inference Speedups", Figure 2): each sequence's cached
 * tokens live in fixed-size pages of a shared pool, found through a page table.
 *   Key pool   k_pages [num_pages, h_k, page_tokens, d] (dtype), one page holds the
 *              rows of every key head for page_tokens consecutive tokens;
 *   value pool v_pages [num_pages, h_v, page_tokens, d_v], with the same page ids;
 *   table [B, max_pages] int32 (device): table[b*max_pages + p] is the page holding
 *              tokens [p*page_tokens, (p+1)*page_tokens) of sequence b.
 * page_tokens is a power of two >= 16; max_pages*page_tokens >= max_l_kv. Entries
 * for tokens < l_kv[b] must lie in [0, num_pages) (a device-side precondition, like
 * l_kv); other entries are never used for results, and every page id the kernels
 * read is clamped into [0, num_pages), so stale entries cannot address memory
 * outside the pools. Logits, thresholds, kept sets, counts and flags equal those of
 * the contiguous calls on the same token rows exactly; outputs agree up to the
 * order of the floating-point sums (the dense call's are identical). */
typedef struct saga_pages {
  const int32_t* table;  /* [B, max_pages] page ids (device) */
  int32_t max_pages;     /* row stride of the table */
  int32_t page_tokens;   /* tokens per page: a power of two, at least 16 */
  int32_t num_pages;     /* pages in each pool */
} saga_pages;

/* saga_decode_attn over paged caches; every other argument as there. s->l_max is
 * only the capacity bound (max_l_kv <= l_max), not a stride. SAGA_ERR_NULL for a
 * NULL pages or table, SAGA_ERR_SHAPE for a bad page size or a table too short
 * for max_l_kv. */
saga_status saga_decode_attn_paged(const saga_shape* s, const saga_pages* pages, const void* q,
                                   const void* k_pages, const void* v_pages, const int32_t* l_kv,
                                   int32_t max_l_kv, int32_t N, int32_t refresh_period, int64_t step,
                                   float* tau, void* out, int32_t* sel_count, int32_t* sel_idx,
                                   int32_t sel_cap, int32_t* flags, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* saga_dense_gqa_attn over paged caches (the dense baseline of the same layout);
 * arguments and errors as in saga_decode_attn_paged and saga_dense_gqa_attn. */
saga_status saga_dense_gqa_attn_paged(const saga_shape* s, const saga_pages* pages, const void* q,
                                      const void* k_pages, const void* v_pages, const int32_t* l_kv,
                                      int32_t max_l_kv, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * A decode layer around the attention step (one new token per sequence), for
 * measuring the step inside a model layer with random weights. Eq. (1) of the
 * summary page ("Attention Mechanism Formalization"): Q = X W_Q, K = X W_K,
 * V = X W_V, with h_k key heads and h_v value heads ("SAGA Architecture"), then the
 * attention and the output projection W_O. Normalisation, rotary embeddings, biases
 * and the residual are the caller's (the pages define none for this step).
 * Weights and activations are bf16, products accumulate in fp32.
 *   x      [B, d_model]                     the new token's hidden state per sequence
 *   w_qkv  [(h_q + h_k + h_v)*d, d_model]   rows: the q features (head-major), then
 *                                           the k features, then the v features
 *                                           (i.e. W_Q, W_K, W_V transposed, stacked)
 *   w_o    [d_model, h_q*d]                 W_O transposed: row o gives output o
 *   y      [B, d_model]                     attn.out_dtype
 * ------------------------------------------------------------------------------ */
typedef enum saga_attention { SAGA_ATTN_ATOPN = 0, SAGA_ATTN_DENSE = 1 } saga_attention;

typedef struct saga_layer {
  saga_shape attn;   /* heads, d, cache capacity l_max, scale; dtype must be SAGA_BF16
                        and d_v 0 or d (one head dimension for q, K and V);
                        out_dtype is the dtype of y (the attention output feeding
                        W_O is bf16) */
  int32_t d_model;   /* hidden size: a multiple of 32 */
} saga_layer;

/* y[b, o] = sum_i x[b, i] * w[o, i]: x [batch, n_in] bf16, w [n_out, n_in] bf16,
 * y [batch, n_out] in out_dtype; fp32 accumulation, bf16 output rounded to nearest
 * even. n_in must be a multiple of 32 (SAGA_ERR_SHAPE otherwise). */
saga_status saga_linear(int32_t batch, int32_t n_in, int32_t n_out, const void* x, const void* w, void* y,
                        int32_t out_dtype, void* stream);

/* Eq. (1) for the new token plus the cache append: q [B, h_q, d] (bf16) = the first
 * h_q*d projections; the next h_k*d and h_v*d projections, rounded to bf16, become
 * row l_kv[b] of every key and value head of sequence b (caches [B, h_k, l_max, d]
 * and [B, h_v, l_max, d]); l_kv_next[b] = l_kv[b] + 1. A full cache (l_kv[b] ==
 * l_max) gets no row and l_kv_next[b] = l_max. l_kv and l_kv_next must be different
 * arrays. */
saga_status saga_qkv_append(const saga_layer* L, const void* x, const void* w_qkv, void* k_cache,
                            void* v_cache, const int32_t* l_kv, int32_t* l_kv_next, void* q,
                            void* stream);

/* Workspace of saga_decode_layer: the attention's workspace (same zero-fill rule,
 * saga_workspace_init) plus the q and attention-output activations. 0 if invalid. */
size_t saga_layer_workspace_bytes(const saga_layer* L, int32_t N, int32_t max_l_kv);

/* One decode layer: saga_qkv_append, then the attention over the l_kv_next[b] rows
 * (attention = SAGA_ATTN_ATOPN: saga_decode_attn with N, refresh_period, step, tau,
 * sel_count and flags as there; SAGA_ATTN_DENSE: saga_dense_gqa_attn, tau, N and
 * the step arguments unused), then y = O W_O with O [B, h_q*d] the bf16 attention
 * output. max_l_kv (host) bounds l_kv_next[] (<= l_max). Every argument is checked
 * before the first launch. */
saga_status saga_decode_layer(const saga_layer* L, int32_t attention, const void* x, const void* w_qkv,
                              const void* w_o, void* k_cache, void* v_cache, const int32_t* l_kv,
                              int32_t* l_kv_next, int32_t max_l_kv, int32_t N, int32_t refresh_period,
                              int64_t step, float* tau, void* y, int32_t* sel_count, int32_t* flags,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * GQA-to-SAGA key-head merge, the closed-form initialisation of a SAGA student from
 * a grouped-query teacher (summary page, section "GQA-to-SAGA Conversion > Stage 1:
 * Closed-Form Initialization"). Teacher key heads are merged in pairs: h_k teacher
 * heads become h_k / 2 student heads, and the query heads of both heads of a pair
 * read the merged head.
 *   eq. (13): L_ab(M) = sum over the query heads j of head a of
 *             ||Q^j (X M)^T - Q^j (X W_K^a)^T||_F^2, plus the same over head b;
 *   Lemma 4.1, eq. (15): the minimiser M_ab = (W_K^a S_a + W_K^b S_b)(S_a + S_b)^+,
 *             S_r = sum over the query heads j of head r of Q^j^T Q^j, Q^j = X W_Q^j;
 *   Theorem 4.2, eq. (14): the pairing is the minimum-weight perfect matching of
 *             the complete graph on the teacher heads with weights L_ab(M_ab).
 * Query head j belongs to teacher key head floor(j * h_k / h_q). The pseudo-inverse
 * treats eigenvalues of S_a + S_b below 1e-5 times the largest as zero. Layouts
 * (row-major, bf16 inputs): x [tokens, d_model] calibration hidden states;
 * w_q [h_q*d, d_model] and w_k [h_k*d, d_model], the transposed projections (row
 * f holds output feature f, head-major, as w_qkv of the decode layer).
 * ------------------------------------------------------------------------------ */
typedef struct saga_merge_shape {
  int32_t tokens;    /* calibration tokens T >= 1 (rows of x) */
  int32_t d_model;   /* hidden size D: a multiple of 32 */
  int32_t h_q;       /* query heads: a multiple of h_k */
  int32_t h_k;       /* teacher key heads: even, 2..16 */
  int32_t d;         /* head dimension: 64 or 128 */
} saga_merge_shape;

/* Workspace bytes of the merge calls (no zero fill needed); 0 if the shape is invalid. */
size_t saga_merge_workspace_bytes(const saga_merge_shape* s);

/* Eq. (13) at eq. (15) for every pair of teacher key heads: loss [h_k, h_k] float32
 * (device), symmetric, zero diagonal. Leaves the coefficients of every pair's merged
 * projection in the workspace for saga_merge_keys. */
saga_status saga_merge_losses(const saga_merge_shape* s, const void* x, const void* w_q, const void* w_k,
                              float* loss, void* workspace, size_t workspace_bytes, void* stream);

/* Theorem 4.2 on the host: the exact minimum-weight perfect matching of n (even,
 * 2..16) vertices, weights w [n, n] (host, row-major; the diagonal is ignored, the
 * rest must be finite). partner [n] (host) receives each vertex's partner; total
 * (host, may be NULL) the matching's weight. Ties go to the matching found first
 * when every vertex is paired with the lowest free one in increasing partner order.
 * Pure host code: no device work. */
saga_status saga_min_weight_pairing(int32_t n, const float* w, int32_t* partner, double* total);

/* Eq. (15) for the pairs of `partner` (host [h_k], partner[partner[a]] == a):
 * w_out [h_k/2 * d, d_model] float32 (device), merged head i = the i-th pair in
 * increasing order of its lower head, row i*d + c = column c of its M. Needs the
 * workspace of a saga_merge_losses call on the same inputs, earlier on `stream`. */
saga_status saga_merge_keys(const saga_merge_shape* s, const void* w_k, const int32_t* partner, float* w_out,
                            void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGA_H */
