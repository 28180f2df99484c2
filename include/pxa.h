/*
 * pxa.h -- C ABI of the MI355X (gfx950) ProxyAttn block-sparse causal prefill
 * attention library (libpxa.so).
 *
 * Method: "ProxyAttn" as described in the ProxyAttn blog post
 * (ir.hit.edu.cn, "ProxyAttn ... ICLR 2026"), section 4 ("ProxyAttn方法详解"):
 *   step 1: pool Q and K over the heads of a group into proxy heads, estimate
 *           token-level proxy scores and max-pool them to 128x128 block scores,
 *           rank the key blocks of each query-block row;
 *   step 2: estimate each head's block budget from the last query block;
 *   final:  turn ranking + budgets into a block-sparse mask and run
 *           FlashAttention-style attention over the kept blocks only.
 * The abstract on the arXiv listing page (mlsanity.com, "ProxyAttn: Guided
 * Sparse Attention via Representative Heads") names the same parts:
 * representative (pooled) heads and block-aware dynamic budget estimation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Causal prefill of one sequence (pxa_prefill_batch: several, one after
 *    another).  H query heads, Hkv KV heads, N tokens, head dimension d, block
 *    B = 128, nb = ceil(N / B) key/query blocks (when B does not divide N the
 *    last block is partial and every step uses the tokens it has), G proxies.
 *  - Query head h uses KV head h / (H / Hkv).  Proxy group g holds query heads
 *    [g*H/G, (g+1)*H/G) and the (contiguous) KV heads those use.
 *  - Q, O: bfloat16 [H][N][d]; K, V: bfloat16 [Hkv][N][d]; all row-major and
 *    contiguous.  Proxies Qbar, Kbar are block-scaled fp16 [G][N][d] with
 *    int32 exponents qexp, kexp [G][nb]: element t of block I of proxy g holds
 *    fp16(mean * 2^exp[g][I]) (see pxa_proxy_pool).  Tensor pointers are
 *    device pointers, 16-byte aligned; int32/fp32 arrays 4-byte aligned;
 *    workspaces 256-byte aligned.
 *  - The caller owns every buffer (inputs, outputs, workspace).  The library
 *    never allocates, frees or synchronises; it enqueues kernels on `stream`
 *    (a hipStream_t; NULL = the null stream) and returns.  Buffers must stay
 *    valid until that stream work completes.  No global mutable state: calls
 *    on different streams with different buffers may run concurrently.
 *  - Return value: PXA_OK (0) or a negative PXA_E* code.  Every argument is
 *    validated on the host before anything is launched, so an error return
 *    means nothing was enqueued, except PXA_EHIP (a launch failed; earlier
 *    kernels of the same call may have been enqueued).  Inputs are assumed
 *    finite (NaN/Inf are not checked).  Results are deterministic for a given
 *    device and inputs.
 */
#ifndef PXA_H
#define PXA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PXA_ABI_VERSION 8

enum {
  PXA_OK = 0,
  PXA_EINVAL = -1,       /* inconsistent shape, grouping, gamma or scale     */
  PXA_EUNSUPPORTED = -2, /* d not 64/128, block not 128, N or H*nb^2 too big   */
  PXA_ENULL = -3,        /* a required pointer is NULL                       */
  PXA_EALIGN = -4,       /* a pointer violates its alignment requirement    */
  PXA_EWORKSPACE = -5,   /* workspace smaller than the *_workspace_bytes query */
  PXA_EHIP = -6          /* a kernel launch failed (see pxa_last_hip_error)  */
};

/* Problem description.  Plain data; the library keeps no pointer to it. */
typedef struct pxa_config {
  int32_t num_heads;     /* H  >= 1                                              */
  int32_t num_kv_heads;  /* Hkv >= 1, H % Hkv == 0                               */
  int32_t seq_len;       /* N, 1 <= N <= 524288; nb = ceil(N/128) blocks, the
                            last one partial when 128 does not divide N; the
                            causal blocks of all heads, H*nb*(nb+1)/2, must fit
                            the int32 CSR (at nb = 4096: H <= 255), else
                            PXA_EUNSUPPORTED                                     */
  int32_t head_dim;      /* d, 64 or 128                                         */
  int32_t block;         /* must be 128 (blog post section 2: 128x128 blocks)    */
  int32_t num_proxies;   /* G: H % G == 0 and (Hkv % G == 0 or G % Hkv == 0)     */
  float gamma;           /* budget threshold, 0 < gamma <= 1                     */
  float softmax_scale;   /* > 0, or <= 0 for 1/sqrt(d)                           */
} pxa_config;

/* Method variants.  Budget: the method's own budget is DYNAMIC (section 4,
 * step 2: the last small portion of the query blocks probes each head's
 * sparsity); FIXED is the one-budget-for-all-heads comparison that step
 * draws; RATIO is the Top-K-by-proportion choice of the XAttention report
 * (leeon-k.github.io, section 2.2).  Scoring: score_stride s > 1 is the
 * sequence-level skip that section 5 credits for the low estimation cost,
 * read as scoring only every s-th query of a block (offsets s-1, 2s-1, ...,
 * B-1; a partial last block adds its last query) against every key -- an
 * approximation of the s = 1 scores.  Every
 * entry point that takes a `const pxa_options*` reads NULL as
 * {PXA_BUDGET_DYNAMIC, 1, 0, 0, 1, 0}, the behaviour of the calls without _ex.
 * Attention: skip_threshold > 0 turns on the running-max skip of the BLASST
 * pages (kept blocks are visited diagonal first, then by descending index; a
 * skipped block costs its QK^T product only). */
enum { PXA_BUDGET_DYNAMIC = 0, PXA_BUDGET_FIXED = 1, PXA_BUDGET_RATIO = 2 };
#define PXA_MAX_PROBE_BLOCKS 64
typedef struct pxa_options {
  int32_t budget_mode;   /* PXA_BUDGET_*                                         */
  int32_t last_blocks;   /* DYNAMIC: m, 1 <= m <= min(nb, PXA_MAX_PROBE_BLOCKS):
                            the masses average every query of the last m blocks */
  int32_t fixed_blocks;  /* FIXED: k >= 1, every head keeps min(k, I+1) ranked
                            blocks of row I (plus the diagonal)                  */
  float ratio;           /* RATIO: 0 < r <= 1, row I keeps ceil(r*(I+1)) ranked
                            blocks (product rounded to fp32 first; at least 1)
                            plus the diagonal, the same for every head           */
  int32_t score_stride;  /* 1, 2 or 4: queries scored per block = B / stride     */
  float skip_threshold;  /* 0: off.  0 < lam <= 1: BLASST running-max skip in the
                            attention (a 32-query group skips a block when
                            exp(block max - running max) < lam for all its
                            queries, scaled logits) -- an approximation          */
} pxa_options;

/* Sizes and offsets of the whole-pipeline workspace (bytes from its start).
 * Intermediates are left there by pxa_prefill so a caller can inspect them. */
typedef struct pxa_workspace_layout {
  size_t qbar;      /* fp16 [G][N][d] (block-scaled)     */
  size_t kbar;      /* fp16 [G][N][d] (block-scaled)     */
  size_t qexp;      /* int32 [G][nb]: exponents of qbar  */
  size_t kexp;      /* int32 [G][nb]: exponents of kbar  */
  size_t scores;    /* fp32 [G][nb][nb]                  */
  size_t masses;    /* fp32 [H][nb]                      */
  size_t k_h;       /* int32 [H]                         */
  size_t row_ptr;   /* int32 [H*nb + 1]                  */
  size_t col_idx;   /* int32 [H*nb*(nb+1)/2] (capacity)  */
  size_t row_order; /* int32 [H*nb]: attention schedule  */
  size_t budget_ws; /* pxa_budget_workspace_bytes        */
  size_t select_ws; /* pxa_select_workspace_bytes        */
  size_t total;     /* == pxa_workspace_bytes            */
} pxa_workspace_layout;

/* ---- queries (host only, no device work) ------------------------------- */
int pxa_abi_version(void);
const char* pxa_strerror(int code);
/* Message of the last HIP error seen by a PXA_EHIP return on this thread. */
const char* pxa_last_hip_error(void);
/* PXA_OK if the configuration is valid, else the code a call would return. */
int pxa_validate_config(const pxa_config* cfg);
/* Whole-pipeline workspace size in bytes; 0 if cfg is invalid. */
size_t pxa_workspace_bytes(const pxa_config* cfg);
int pxa_get_workspace_layout(const pxa_config* cfg, pxa_workspace_layout* out);
/* Scratch needed by pxa_budget_estimate / pxa_block_select; 0 if invalid. */
size_t pxa_budget_workspace_bytes(const pxa_config* cfg);
size_t pxa_select_workspace_bytes(const pxa_config* cfg);
/* Capacity col_idx must have: H * nb * (nb + 1) / 2 entries (every causal block). */
size_t pxa_max_col_entries(const pxa_config* cfg);
/* PXA_OK if cfg and opts (NULL: the defaults) are valid together, else the
 * code a call would return (PXA_EINVAL for a bad mode or parameter). */
int pxa_validate_options(const pxa_config* cfg, const pxa_options* opts);
/* The _ex queries size the workspaces for a variant (a probe of m blocks
 * needs m times the budget scratch); 0 if cfg or opts is invalid. */
size_t pxa_workspace_bytes_ex(const pxa_config* cfg, const pxa_options* opts);
int pxa_get_workspace_layout_ex(const pxa_config* cfg, const pxa_options* opts,
                                pxa_workspace_layout* out);
size_t pxa_budget_workspace_bytes_ex(const pxa_config* cfg, const pxa_options* opts);

/* ---- the pipeline ------------------------------------------------------- */

/* Whole method on one layer: proxy pool -> proxy scores -> budgets -> block
 * selection -> block-sparse attention.  q/k/v inputs, o output (layouts
 * above); ws of at least pxa_workspace_bytes(cfg) bytes, laid out as
 * pxa_get_workspace_layout reports. */
int pxa_prefill(const pxa_config* cfg, const void* q, const void* k, const void* v,
                void* o, void* ws, size_t ws_bytes, void* stream);
/* The same with method variants (NULL: as pxa_prefill); ws of at least
 * pxa_workspace_bytes_ex(cfg, opts) bytes.  FIXED writes k_h and leaves the
 * masses unwritten; RATIO writes neither (budget stage skipped). */
int pxa_prefill_ex(const pxa_config* cfg, const pxa_options* opts, const void* q,
                   const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                   void* stream);

/* The whole method with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): as pxa_prefill_ex, with the workspace in
 * a static array of PXA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  The call allocates and frees
 * nothing.  It works on the current device (the stream must belong to it); its
 * first call on a device looks the array's address up.  PXA_EWORKSPACE, before
 * any device work, when pxa_workspace_bytes_ex(cfg, opts) exceeds the array
 * (64 MiB: up to 28,883 tokens of a 32-head, 8-KV-head, d = 128 layer with
 * four proxies).  Every call on one GPU shares that GPU's array, and the
 * array keeps the last call's intermediates (every one is written before it
 * is read, so nothing needs clearing): calls that overlap in time on one GPU,
 * on different streams or threads, race and must be serialised by the
 * caller. */
#define PXA_NOALLOC_SCRATCH_BYTES (64u << 20)
int pxa_prefill_noalloc(const pxa_config* cfg, const pxa_options* opts, const void* q,
                        const void* k, const void* v, void* o, void* stream);

/* Several sequences in one call (batched / packed varlen prefill, equal or
 * different lengths).  Sequence s has seq_lens[s] tokens (host array; each in
 * [1, cfg->seq_len]); its tensors are the usual per-sequence blocks
 * Q/O [H][N_s][d], K/V [Hkv][N_s][d], stored one after another (sequence s
 * starts after the elements of sequences 0..s-1).  Each sequence's output
 * equals what pxa_prefill_ex gives for it alone.
 *   Fused (ws_bytes >= pxa_batch_workspace_bytes): the sequences are taken in
 * groups of up to PXA_MAX_FUSED_SEQS consecutive ones and each group runs as
 * one set of launches (one grid per stage over every block of every sequence
 * of the group, one CSR and one attention schedule for the whole group), so
 * many short sequences fill the GPU together.  The workspace then holds the
 * last group's intermediates, laid out as pxa_get_batch_workspace_layout
 * gives for that group.
 *   Otherwise (ws_bytes >= pxa_workspace_bytes_ex(cfg, opts), cfg->seq_len
 * the longest length): one sequence at a time, the workspace holding the last
 * sequence's intermediates.
 * PXA_EINVAL for num_seqs < 1, a length outside [1, cfg->seq_len] or a probe
 * longer than a sequence, PXA_ENULL for a NULL seq_lens, PXA_EWORKSPACE below
 * both sizes.  Every length is checked before the first launch. */
#define PXA_MAX_FUSED_SEQS 64
/* Workspace bytes for the fused batch path: the largest group's; 0 if
 * cfg, opts or the lengths are invalid. */
size_t pxa_batch_workspace_bytes(const pxa_config* cfg, const pxa_options* opts,
                                 int32_t num_seqs, const int32_t* seq_lens);
/* Layout of the fused workspace of a batch that forms one group (at most
 * PXA_MAX_FUSED_SEQS sequences): every part is the concatenation of the
 * sequences' own parts in order (qbar/kbar [G][N_s][d] each, qexp/kexp
 * [G][nb_s] each, scores [G][nb_s][nb_s] each, masses [H][nb_s] each, k_h [H] each, then one CSR
 * over all rows -- sequence s's H*nb_s rows after those of the sequences
 * before it, column indices local to the sequence -- and one row_order over
 * those rows).  PXA_EINVAL if the batch forms more than one group. */
int pxa_get_batch_workspace_layout(const pxa_config* cfg, const pxa_options* opts,
                                   int32_t num_seqs, const int32_t* seq_lens,
                                   pxa_workspace_layout* out);
int pxa_prefill_batch(const pxa_config* cfg, const pxa_options* opts, int32_t num_seqs,
                      const int32_t* seq_lens, const void* q, const void* k, const void* v,
                      void* o, void* ws, size_t ws_bytes, void* stream);

/* Step 1, head pooling (blog post section 4, step 1 "Head Pooling"; section 3
 * calls it a simple pooling).  The proxy means are qbar = mean of q over the
 * group's query heads and kbar = mean of k over the group's KV heads (fp32
 * sums in head order, IEEE division).  They are stored block-scaled: for proxy
 * g and block I, exp[g][I] = e is the integer that puts the block's largest
 * |mean| in [2^14, 2^15) (0 for an all-zero block), and every element of the
 * block is stored as fp16(mean * 2^e), rounded to nearest even.  qbar, kbar:
 * fp16 [G][N][d] (16-byte aligned); qexp, kexp: int32 [G][nb]. */
int pxa_proxy_pool(const pxa_config* cfg, const void* q, const void* k,
                   void* qbar, void* kbar, int32_t* qexp, int32_t* kexp, void* stream);

/* Step 1, score estimation (section 4, step 1 "Score Estimation": token-level
 * proxy scores, block max-pool, the QK product fused with the pooling).
 * scores[g][I][J] = scale * max over causal token pairs (i in block I,
 * j in block J, j <= i) of qbar[g][i] . kbar[g][j], fp32, for J <= I; -inf
 * for J > I, where qbar, kbar are the proxy values of pxa_proxy_pool (the
 * stored fp16 times 2^-exp).  fp16 MFMA products, fp32 accumulation; the
 * tile max is multiplied by 2^-(qexp[g][I] + kexp[g][J]) and the scale. */
int pxa_proxy_score(const pxa_config* cfg, const void* qbar, const void* kbar,
                    const int32_t* qexp, const int32_t* kexp, float* scores, void* stream);
/* The same with the sequence-level skip: opts->score_stride = s scores only
 * the queries at offsets s-1, 2s-1, ..., B-1 of each query block (every key
 * of the causal range); s = 1 (or NULL opts) is pxa_proxy_score. */
int pxa_proxy_score_ex(const pxa_config* cfg, const pxa_options* opts, const void* qbar,
                       const void* kbar, const int32_t* qexp, const int32_t* kexp,
                       float* scores, void* stream);

/* Step 2, dynamic budget (section 4, step 2: the last query block estimates
 * each head's block-level sparsity; the abstract's "block-aware dynamic budget
 * estimation").  For head h: masses[h][J] = mean over the queries of the last
 * query block (B of them, fewer when it is partial) of their exact causal
 * softmax mass in key block J (fp32); k_h[h] = smallest k
 * such that the masses of the first k blocks of the group's ranking of row
 * nb-1 (score descending, block ascending on ties) sum to >= gamma, else nb.
 * scores: as written by pxa_proxy_score.  ws: pxa_budget_workspace_bytes. */
int pxa_budget_estimate(const pxa_config* cfg, const void* q, const void* k,
                        const float* scores, int32_t* k_h, float* masses,
                        void* ws, size_t ws_bytes, void* stream);
/* Budget variants of step 2.  DYNAMIC with m probe blocks: as above with the
 * masses averaged over every query of the last m blocks (each over its own
 * causal keys);
 * ws: pxa_budget_workspace_bytes_ex.  FIXED: k_h[h] = fixed_blocks for every
 * head; only k_h is used (q, k, scores, masses, ws may be NULL).  RATIO has no
 * per-head budget: PXA_EINVAL. */
int pxa_budget_estimate_ex(const pxa_config* cfg, const pxa_options* opts, const void* q,
                           const void* k, const float* scores, int32_t* k_h, float* masses,
                           void* ws, size_t ws_bytes, void* stream);

/* Step 1 ranking + final mask (section 4, step 1 "Block Ranking" with TopK,
 * and the final block sparse mask handed to FlashAttention).  Row (h, I)
 * keeps the first min(k_h[h], I+1) blocks of the group's ranking of row I
 * plus the diagonal block I (k_h < 0 is read as 0).  Output is CSR over rows
 * r = h*nb + I: row_ptr[H*nb+1], col_idx[row_ptr[r] .. row_ptr[r+1])
 * ascending.  col_idx needs pxa_max_col_entries(cfg) capacity.
 * row_order (may be NULL): receives a permutation of the H*nb rows, the
 * schedule for pxa_sparse_prefill (it never changes any result).  Position p
 * is meant for XCD p mod 8 (workgroups are dealt to the 8 XCDs round-robin):
 * XCD x gets the rows whose midpoint in the cumulative work row_ptr lies in
 * the x-th eighth (a contiguous range of rows, hence of KV heads, so their
 * K/V tiles stay in that XCD's L2), longest first; when that is more rows
 * than it has positions, its shortest rows fill other XCDs' spare positions.
 * Rows of equal length come in no fixed order.
 * ws: pxa_select_workspace_bytes. */
int pxa_block_select(const pxa_config* cfg, const float* scores, const int32_t* k_h,
                     int32_t* row_ptr, int32_t* col_idx, int32_t* row_order, void* ws,
                     size_t ws_bytes, void* stream);
/* The same with a budget variant: RATIO keeps, in every head, the first
 * ceil(fl32(ratio * (I+1))) (at least 1, at most I+1) blocks of row I's
 * ranking plus the diagonal, and ignores k_h (which may be NULL); DYNAMIC and
 * FIXED use k_h as pxa_block_select does. */
int pxa_block_select_ex(const pxa_config* cfg, const pxa_options* opts, const float* scores,
                        const int32_t* k_h, int32_t* row_ptr, int32_t* col_idx,
                        int32_t* row_order, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse causal attention over the CSR mask (section 4, final step; the
 * attention of section 2).  o[h][i] = sum of softmax(scale * q.k_j) v_j over
 * the keys j <= i of the kept blocks of row (h, i / B), renormalised over
 * them; fp32 online softmax, bf16 MFMA products, bf16 output (RNE).  Columns
 * of a row must be ascending (as pxa_block_select writes them; otherwise the
 * output is unspecified, though every memory access stays inside the tensors).
 * Entries of a row outside [0, I] are ignored; a row with no valid entry yields
 * zeros.
 * row_order (may be NULL): the order in which rows are handed to the GPU, a
 * permutation of [0, H*nb) such as pxa_block_select writes (entries outside
 * that range are skipped; a repeated row is computed twice with the same
 * result).  NULL: query blocks from last to first, heads rotated so every
 * head visits every XCD. */
int pxa_sparse_prefill(const pxa_config* cfg, const void* q, const void* k, const void* v,
                       const int32_t* row_ptr, const int32_t* col_idx,
                       const int32_t* row_order, void* o, void* stream);
/* The same with opts->skip_threshold (other fields are not used). */
int pxa_sparse_prefill_ex(const pxa_config* cfg, const pxa_options* opts, const void* q,
                          const void* k, const void* v, const int32_t* row_ptr,
                          const int32_t* col_idx, const int32_t* row_order, void* o,
                          void* stream);

/* Dense causal attention with the same kernel (every block J <= I kept):
 * the baseline the sparse path is measured against. */
int pxa_dense_prefill(const pxa_config* cfg, const void* q, const void* k, const void* v,
                      void* o, void* stream);
/* Dense causal attention with the running-max skip (BLASST on its own). */
int pxa_dense_prefill_ex(const pxa_config* cfg, const pxa_options* opts, const void* q,
                         const void* k, const void* v, void* o, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PXA_H */
