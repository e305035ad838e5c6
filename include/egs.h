/*
 * egs.h -- C ABI of the entropy-guided, head-adaptive sparse attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * Method sources (cited by page title and section / equation / algorithm):
 *   [EI] "From Rigid to Dynamic: Entropy-Guided Adaptive Inference for
 *        Long-Context LLMs" (EntropyInfer), arXiv 2606.09508.
 *   [KV] Blog notes "attention-kv-cache-mechanics", InfoKV part (eq. 4
 *        window-mean attention score, eq. 8 fused score).
 *   [EP] "EntroPrefill: Renyi-Guided Context Pruning with Conditional Stability
 *        Guarantees for Retrieval-Augmented Generation".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Ownership: every tensor pointer is a caller-owned DEVICE buffer.  The
 *    library never allocates or frees device memory; scratch space is passed
 *    in through `workspace` arguments sized by the *_workspace() queries.
 *  - Layout: tensors are dense, row-major, head-major, exactly as given in the
 *    comments ([Hq, N, d] means index (h * N + n) * d + i).
 *  - Element types: `dtype` (EGS_BF16 or EGS_F32) applies to q, k, v, outputs
 *    and caches; scores, entropies and log-sum-exps are float32; indices and
 *    budgets are int32; head classes are int8.
 *  - Alignment: q / k / v / out / cache pointers must be 16-byte aligned.
 *  - Asynchrony: work is enqueued on `stream`; EGS_OK means "enqueued".
 *    Outputs are valid once the caller synchronizes the stream.  No call
 *    blocks the host or copies data to it.
 *  - Errors: all argument checks run on the host before anything is
 *    launched, so a call that fails launches nothing.  Invalid shapes or null
 *    required pointers give EGS_EINVAL; shapes outside the kernels' supported
 *    range give EGS_ENOTSUP; an undersized workspace gives EGS_EWORKSPACE; a
 *    failed launch gives EGS_EHIP.  egs_last_error() returns a thread-local
 *    message describing the last failure of the calling thread.
 *  - Thread safety: calls are stateless apart from the thread-local error
 *    message; concurrent calls on different streams with distinct output
 *    buffers are independent.
 *  - GQA: query head h reads KV head g(h) = h / (Hq / Hkv) (contiguous groups).
 *  - Softmax scale: sm_scale = 0 selects 1/sqrt(head_dim) ([EI] Sec. 2).
 */
#ifndef EGS_H_
#define EGS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EGS_ABI_VERSION 7

typedef enum {
  EGS_OK = 0,
  EGS_EINVAL = 1,
  EGS_ENOTSUP = 2,
  EGS_EWORKSPACE = 3,
  EGS_EHIP = 4
} egs_status;

typedef enum { EGS_BF16 = 0, EGS_F32 = 1 } egs_dtype;

/* Shannon entropy, or Renyi entropy of order renyi_alpha ([EP] Sec. 3.1). */
typedef enum { EGS_SHANNON = 0, EGS_RENYI = 1 } egs_entropy_kind;

/* How key blocks are represented for the observation rows.
 * MEAN_PROBE: mean of every key block, scored against the last probe_len
 *   queries of each segment.
 * MAXMIN: the max / min representatives of [EI] Sec. 4.2 Alg. 1-2 (whole
 *   segments of queries, whole blocks of keys; probe_len is not used). */
typedef enum { EGS_POOL_MEAN_PROBE = 0, EGS_POOL_MAXMIN = 1 } egs_pool_kind;

/* Budget policy ([EI] Sec. 1: rigid heads get a fixed minimal budget, dynamic
 * heads more; [EI] Sec. 4.2 Alg. 3: budget driven by the entropy fluctuation
 * between adjacent segments). */
typedef enum {
  EGS_BUDGET_FIXED = 0,        /* k = kclamp(frac * C_B(s))                               */
  EGS_BUDGET_TWO_LEVEL = 1,    /* frac_rigid for rigid heads, frac_dynamic otherwise      */
  EGS_BUDGET_PROPORTIONAL = 2, /* f = min(frac_max, max(frac_min, frac_max*E/ln C_B(s)))  */
  EGS_BUDGET_ALG3 = 3          /* Alg. 3 with base budget base_tokens (tokens)            */
} egs_budget_mode;

/* Prefill problem ([EI] Sec. 4.1 notation).
 *   N = seq_len, L_S = segment_size, L_B = block_size, P = probe_len.
 *   C_S = N / L_S segments, C_B = N / L_B key blocks, and segment s sees the
 *   C_B(s) = (s + 1) * L_S / L_B causal key blocks 0 .. C_B(s)-1.
 * Valid shapes: N % L_S == 0, L_S % L_B == 0, 1 <= P <= L_S,
 *   n_q_heads % n_kv_heads == 0, head_dim in {16, 32, 64, 128}, L_B % 16 == 0,
 *   16 <= L_B <= 256, C_B <= 16384. */
typedef struct {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t seq_len;
  int32_t block_size;
  int32_t segment_size;
  int32_t probe_len;
  int32_t dtype;      /* egs_dtype */
  float sm_scale;     /* 0 => 1/sqrt(head_dim) */
} egs_prefill_shape;

typedef struct {
  int32_t mode;              /* egs_budget_mode */
  double frac;               /* FIXED */
  double frac_rigid;         /* TWO_LEVEL */
  double frac_dynamic;       /* TWO_LEVEL */
  double frac_min;           /* PROPORTIONAL */
  double frac_max;           /* PROPORTIONAL */
  double entropy_threshold;  /* e_t: rigid(h) <=> max_s E[h,s] < e_t (all modes) */
  double base_tokens;        /* ALG3: B_h in tokens */
  double alg3_alpha;         /* ALG3: budget coefficient (0.5 in the paper) */
  double alg3_delta_t;       /* ALG3: fluctuation threshold (0.4 in the paper) */
} egs_budget_policy;

/* ---------------------------------------------------------------------------
 * Step 1-5: observation rows and their entropy.
 * [EI] Sec. 4.2 (observation attention over blocks, then "each row's
 * attention entropy"); [KV] eq. 4 and [EP] Sec. 2.1 (mean of the attention
 * rows of a window of queries); [EP] Sec. 3.1 (Renyi order).
 *
 *   kbar[g, j]       = mean of keys j*L_B .. (j+1)*L_B-1 of KV head g
 *   z[h, s, u, j]    = sm_scale * q[h, u] . kbar[g(h), j],
 *                      u in the last P positions of segment s, j < C_B(s)
 *   block_scores[h, s, j] = (1/P) * sum_u softmax_j(z[h, s, u, :])[j]
 *                           for j < C_B(s), and -1 for j >= C_B(s)
 * With pool_kind EGS_POOL_MAXMIN ([EI] Sec. 4.2 Alg. 1-2) instead:
 *   Qx[h, s] / Qn[h, s] = element-wise max / min of q[h, u] over the L_S
 *                      positions u of segment s
 *   Kx[g, j] / Kn[g, j] = element-wise max / min of the keys of block j
 *   S1..S4           = softmax_j over j < C_B(s) of sm_scale * (Qx.Kx_j,
 *                      Qx.Kn_j, Qn.Kx_j, Qn.Kn_j)
 *   block_scores[h, s, j] = A_j / sum_j' A_j',
 *                      A_j = max((S1_j + S2_j) / 2, (S3_j + S4_j) / 2)
 *   (Alg. 2 leaves out sm_scale and the renormalisation; both are applied.)
 *
 *   entropy[h, s]    = -sum_j a ln a        (EGS_SHANNON)
 *                    = ln(sum_j a^alpha)/(1-alpha)   (EGS_RENYI, alpha > 0,
 *                      alpha == 1 means Shannon)
 *
 *   q: [Hq, N, d] dtype     k: [Hkv, N, d] dtype        (read only)
 *   block_scores: [Hq, C_S, C_B] float32 (written)
 *   entropy:      [Hq, C_S]      float32 (written)
 *   workspace: >= egs_entropy_score_workspace(shape) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
size_t egs_entropy_score_workspace(const egs_prefill_shape* shape);
egs_status egs_entropy_score(const egs_prefill_shape* shape, int32_t pool_kind,
                             int32_t entropy_kind, float renyi_alpha,
                             const void* q, const void* k,
                             float* block_scores, float* entropy,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * egs_entropy_score without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid hipMalloc).  Same arguments, checks, kernels and results as
 * egs_entropy_score; the scratch is a fixed device array of
 * EGS_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  A shape whose egs_entropy_score_workspace() exceeds that
 * size returns EGS_EWORKSPACE before anything is launched (the 131072-token,
 * 32 / 8-head layer needs 22 MiB).  The call allocates nothing: no hipMalloc,
 * no hipFree, no allocating library routine.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  No part of the array
 * has to start at zero; it keeps the last call's contents.
 * ------------------------------------------------------------------------- */
#define EGS_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
egs_status egs_entropy_score_static(const egs_prefill_shape* shape, int32_t pool_kind,
                                    int32_t entropy_kind, float renyi_alpha,
                                    const void* q, const void* k,
                                    float* block_scores, float* entropy,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Steps 6-7: classify heads and allocate per-(head, segment) budgets.
 * [EI] Sec. 4.2 Alg. 3 (rigid test on the maximum segment entropy; budget
 * recurrence with clamp to [B_h, 3 B_h] and a divisor guarded by e_t).
 *
 *   head_is_rigid[h] = max_s entropy[h, s] < e_t               ([Hq] int8)
 *   budget[h, s]     = kclamp(x) = min(C_B(s), max(1, ceil(x - 1e-9))) with
 *                      x = frac * C_B(s) (FIXED / TWO_LEVEL / PROPORTIONAL) or
 *                      x = B_s / L_B (ALG3), computed in float64.
 *   entropy: [Hq, C_S] float32 (read);  budget: [Hq, C_S] int32 (written).
 * ------------------------------------------------------------------------- */
egs_status egs_allocate_budget(const egs_prefill_shape* shape,
                               const egs_budget_policy* policy,
                               const float* entropy, int8_t* head_is_rigid,
                               int32_t* budget, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Step 8: top-k key-block selection ([EI] App. A eq. (2): top-k blocks per
 * segment; ties go to the lower block index).
 *
 *   Sel(h, s) = the k = min(budget[h, s], C_B(s), k_max) blocks j < C_B(s)
 *   with the largest block_scores[h, s, j], order (score desc, index asc).
 *   block_idx: [Hq, C_S, k_max] int32, ascending, padded with -1 (written)
 *   block_cnt: [Hq, C_S] int32 = k (written)
 * ------------------------------------------------------------------------- */
egs_status egs_select_blocks(const egs_prefill_shape* shape,
                             const float* block_scores, const int32_t* budget,
                             int32_t k_max, int32_t* block_idx,
                             int32_t* block_cnt, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Steps 1-8 in one call: egs_entropy_score, egs_allocate_budget and
 * egs_select_blocks with the same arguments, checks and bit-identical
 * outputs ([EI] Sec. 4.2, Alg. 3 and App. A eqs. (1)-(2)), enqueued as
 * fewer kernels: the entropies, head classes and budgets are formed inside
 * the selection kernel (each (head, segment) workgroup recomputes its head's
 * entropies from the scoring pass's partial sums), so no separate entropy or
 * budget launch follows the scoring kernels.
 *   workspace: >= egs_entropy_score_workspace(shape) bytes, 256-byte aligned.
 *   Outputs as the three calls: block_scores, entropy, head_is_rigid, budget,
 *   block_idx, block_cnt.
 * ------------------------------------------------------------------------- */
egs_status egs_score_select(const egs_prefill_shape* shape, int32_t pool_kind,
                            int32_t entropy_kind, float renyi_alpha,
                            const egs_budget_policy* policy, const void* q, const void* k,
                            int32_t k_max, float* block_scores, float* entropy,
                            int8_t* head_is_rigid, int32_t* budget, int32_t* block_idx,
                            int32_t* block_cnt, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Steps 9-10: block-sparse causal GQA attention over the selected blocks.
 * [EI] App. A eq. (3) (attention over the selected blocks of every segment);
 * [EP] Sec. 2.1 (causal GQA softmax).
 *
 * Query block b (rows b*L_B .. (b+1)*L_B-1) of segment s = b*L_B / L_S attends
 * the blocks L(h, b) = { j in block_idx[h, s, 0 .. cnt-1] : 0 <= j < b } U { b },
 * the own block b causally masked (key t <= row i).  Entries outside 0..b-1
 * are skipped, so any list is safe; a block listed twice is attended twice
 * (egs_select_blocks writes ascending lists without repeats).
 *   out[h, i, :] = sum_t softmax_t(sm_scale * q[h,i] . k[g,t]) v[g,t]
 *   lse[h, i]    = ln sum_t exp(sm_scale * q[h,i] . k[g,t])   (nullable)
 *   q: [Hq, N, d], k, v: [Hkv, N, d], out: [Hq, N, d] (dtype); lse [Hq, N] f32.
 *   workspace: >= egs_sparse_prefill_attn_workspace(shape) bytes, 256-byte
 *   aligned (the bf16 MFMA path packs V into d-major tiles there, Hkv*N*d*2
 *   bytes, followed by 8 KB of work-queue counters that the call
 *   resets itself; other paths need none and accept NULL).  Calls that
 *   share a workspace must not overlap in time (one stream orders them).
 * ------------------------------------------------------------------------- */
size_t egs_sparse_prefill_attn_workspace(const egs_prefill_shape* shape);
egs_status egs_sparse_prefill_attn(const egs_prefill_shape* shape,
                                   const void* q, const void* k, const void* v,
                                   const int32_t* block_idx,
                                   const int32_t* block_cnt, int32_t k_max,
                                   void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode-time KV retention.
 * [EI] Sec. 4.3 and App. B Alg. 4 (score cache entries with a window of the
 * most recent queries, keep the top B_d, gather the kept K/V);
 * [KV] eq. 4 (window mean) and eq. 8 (fusion with softmax of token entropy);
 * [EP] Sec. 2.1 (observer-pooled measure), Sec. 3.1 (sink-isolated entropy,
 * regularized head weights w_h = zeta/r + (1-zeta) softmax_h(-H_h/tau)),
 * Sec. 8.1 (compaction keeps token order).
 *
 * Valid shapes: W = n_obs, 1 <= W <= min(cache_len, 128); n_sink, n_recent,
 * n_keep >= 0; head_dim in {64, 128}; Hq / Hkv <= 16; cache_len <= 2^26.
 * n_total = cache_len if n_sink + n_recent + n_keep >= cache_len, else
 * n_sink + n_keep + n_recent (see egs_kv_retain_total()).
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t cache_len;   /* L */
  int32_t n_obs;       /* W: observers are the queries at positions L-W .. L-1 */
  int32_t n_sink;      /* positions 0 .. n_sink-1 are always kept */
  int32_t n_recent;    /* positions L-n_recent .. L-1 are always kept */
  int32_t n_keep;      /* top entries kept from [n_sink, L - n_recent) */
  int32_t dtype;       /* egs_dtype (only EGS_BF16 is supported) */
  float sm_scale;      /* 0 => 1/sqrt(head_dim) */
} egs_decode_shape;

typedef struct {
  int32_t entropy_kind;    /* egs_entropy_kind for the head entropy H_h */
  float renyi_alpha;       /* Renyi order when entropy_kind == EGS_RENYI */
  double zeta;             /* group floor, in (0, 1] */
  double tau;              /* entropy temperature, > 0 */
  int32_t raw_logit_mode;  /* 1: score = sum of raw scaled logits, as Alg. 4 */
  double info_alpha;       /* InfoKV fusion weight; 1 (or token_entropy NULL) = off */
} egs_retain_params;

int32_t egs_kv_retain_total(const egs_decode_shape* shape);
size_t egs_kv_retain_workspace(const egs_decode_shape* shape);

/*   q_obs:   [B, Hq, W, d] dtype      k_cache, v_cache: [B, Hkv, L, d] dtype
 *   token_entropy: [B, L] float32 or NULL (InfoKV fusion input E_tok)
 *   keep_idx: [B, Hkv, n_total] int32, ascending (written)
 *   k_out, v_out: [B, Hkv, n_total, d] dtype (written; both NULL to skip the gather)
 *   head_entropy: [B, Hq] float32 or NULL (sink-isolated H_h; 0 in raw mode)
 *   scores: [B, Hkv, L] float32 or NULL (the group score mu_t)
 *   workspace: >= egs_kv_retain_workspace(shape) bytes, 256-byte aligned.
 *
 * Score of entry t in group g (mu_t), observer u at position p_u = L-W+u:
 *   A^h_{u,t} = softmax_{t <= p_u}(sm_scale q_{h,u} . k_{g,t}),
 *   a^h_t = (1/W) sum_u A^h_{u,t},  H_h = entropy of a^h restricted to
 *   t >= n_sink and renormalised,  w_h as above,  mu_t = sum_{h in g} w_h a^h_t,
 *   then mu <- info_alpha mu + (1 - info_alpha) softmax_t(E_tok) if fused.
 *   Raw mode: mu_t = sum_{h in g} sum_u sm_scale q_{h,u} . k_{g,t}.
 * keep = sinks U top-n_keep of [n_sink, L-n_recent) under (mu desc, t asc)
 *        U recent, ascending. */
egs_status egs_kv_retain(const egs_decode_shape* shape,
                         const egs_retain_params* params, const void* q_obs,
                         const void* k_cache, const void* v_cache,
                         const float* token_entropy, int32_t* keep_idx,
                         void* k_out, void* v_out, float* head_entropy,
                         float* scores, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode attention of one new token over the kept entries ([EI] App. B Alg. 4
 * output used for generation; no mask: every kept entry precedes the token).
 *   q_new: [B, Hq, d]; k_kept, v_kept: [B, Hkv, n_total, d]; out: [B, Hq, d]
 *   (dtype).  workspace >= egs_sparse_decode_attn_workspace(shape, n_total).
 * ------------------------------------------------------------------------- */
size_t egs_sparse_decode_attn_workspace(const egs_decode_shape* shape,
                                        int32_t n_total);
egs_status egs_sparse_decode_attn(const egs_decode_shape* shape,
                                  const void* q_new, const void* k_kept,
                                  const void* v_kept, int32_t n_total,
                                  void* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Chunk pruning of one prompt ([EP] Sec. 2.1, 3.1-3.2, 4.1-4.2).
 * The prompt's candidate chunks c_i = [begin_i, end_i) (disjoint, ascending,
 * before the W observer positions T-W .. T-1) may be removed; everything else
 * is protected.
 *   pooled measure mu_t = (1/G) sum_g sum_{h in g} w_h a^h_t: window means of
 *     the observers' causal attention rows, Renyi-2 sink-isolated head
 *     entropies, w_h = zeta/r + (1-zeta) softmax(-H/tau)   (Sec. 2.1, 3.1)
 *   p = mu on the candidate tokens, renormalised; pi_i = n_i / N;
 *   M_i = sum_{c_i} p;  p_hat_ij = (p_j + eps_s pi_i/n_i) / (M_i + eps_s pi_i);
 *   l_i = (M_i + eps_s pi_i) / ((1 + eps_s) pi_i);
 *   kappa_i = -H_2(p_hat_i) / ln n_i (0 for n_i = 1);
 *   priority S_i = ln l_i + lambda kappa_i                     (Sec. 3.2)
 *   row masses m[i][a] = sum_{t in c_i} A_{a,t}, rows a = h*W + u
 *   greedy: chunks by (S_i ascending, n_i descending, index ascending), one
 *     scan; chunk i is removed only if every row keeps sum_{E} m[., a] <= eps
 *     and |E| <= k - m0; the scan stops once `target` tokens are removed
 *                                                               (Sec. 4.2)
 * shape: batch 1, cache_len T, n_obs W, n_sink (and the heads); its n_keep
 * and n_recent are not used.  q_obs [Hq, W, d], k [Hkv, T, d] bf16 (device).
 * chunk_bounds: device int32 [n_chunks][2] (begin, end), checked on the
 * device: when the chunks are not ascending, disjoint, non-empty and before
 * the observers, the call removes nothing and sets removed_tokens to -1 and
 * every priority to NaN (every access stays in bounds whatever the values).
 * Outputs (device): removed [k] int8, removed_tokens [1] int32, priority [k]
 * float32, row_mass [k][Hq*W] float32 or NULL.  Valid: 1 <= n_chunks <= 4096,
 * Hq*W <= 8192, eps_s > 0, lambda >= 0, eps >= 0, m0 >= 0, target >= 0.
 * Nothing is copied from host memory, so the call can be captured in a graph.
 * ------------------------------------------------------------------------- */
typedef struct {
  double eps_s;     /* null smoothing epsilon_s > 0 */
  double lambda;    /* concentration weight >= 0 */
  double eps;       /* deletion budget of every observer row (epsilon_a) */
  int32_t m0;       /* at least m0 chunks stay */
  int32_t target;   /* stop once this many tokens are removed */
  double zeta;      /* head-weight floor in (0, 1] */
  double tau;       /* head-weight temperature > 0 */
} egs_prune_params;

size_t egs_chunk_prune_workspace(const egs_decode_shape* shape, int32_t n_chunks);
egs_status egs_chunk_prune(const egs_decode_shape* shape, const egs_prune_params* params,
                           const void* q_obs, const void* k, const int32_t* chunk_bounds,
                           int32_t n_chunks, int8_t* removed, int32_t* removed_tokens,
                           float* priority, float* row_mass, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Optimality-gap certificate of a chunk removal ([EP] Sec. 4.2):
 *   U(y, t) = eps sum_a y_a + t (k - m0) + sum_i [n_i - sum_a y_a m[i][a] - t]_+
 * For prices y_a >= 0 (one per observer row) and t >= 0, U bounds the tokens
 * that any removal set keeping every row within eps and at most k - m0
 * chunks can remove; U - removed_tokens bounds the greedy scan's shortfall.
 * chunk_bounds: device int32 [n_chunks][2] (begin, end); only the lengths
 * n_i = end - begin are used (as given: they are not checked).  Device:
 * row_mass [n_chunks][n_rows] float32 (the egs_chunk_prune output),
 * row_price [n_rows] float32, certificate [1] float64.  Computed in float64.
 * Valid: 1 <= n_chunks <= 4096, 1 <= n_rows <= 8192, eps >= 0, t >= 0,
 * m0 >= 0.  The prices are not checked (device memory): with a negative
 * price U is no bound.  workspace >= egs_prune_certificate_workspace(n_chunks)
 * bytes.
 * ------------------------------------------------------------------------- */
size_t egs_prune_certificate_workspace(int32_t n_chunks);
egs_status egs_prune_certificate(const int32_t* chunk_bounds, int32_t n_chunks, int32_t n_rows,
                                 const float* row_mass, const float* row_price, double eps,
                                 int32_t m0, double t, double* certificate, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Latent decoding ([EI] Sec. 4.3 and App. B: compress the cache only after
 * N_D tokens have been generated, with an observation window that holds the
 * generated tokens' queries; [KV] InfoKV: compress again every fixed number of
 * generated tokens).  One call per generated token:
 *   1. append: k_new / v_new [B, Hkv, d] become entry state->length of every
 *      (b, g) row of k_cache / v_cache; q_new [B, Hq, d] enters the window
 *      q_window [B, Hq, W, d] (its rows move up by one; W = n_obs);
 *   2. out [B, Hq, d] = attention of q_new over entries 0 .. length (the new
 *      entry included, no mask: every entry precedes or is the new token);
 *   3. generated += 1; if generated == n_delay, or interval > 0, generated >
 *      n_delay and (generated - n_delay) % interval == 0: the egs_kv_retain
 *      rule (params; sinks, n_keep, recent of the shape) with the window as the
 *      observers of the last W entries; the kept entries are compacted, in
 *      order, to positions 0 .. n_total-1 and length becomes n_total
 *      (keep_idx, if not NULL, receives the kept positions [B, Hkv, n_total]
 *      in the pre-compression numbering; compressed is set to 1).
 * The shape's cache_len is the capacity C of k_cache / v_cache [B, Hkv, C, d]
 * (bf16).  The caller fills q_window with the queries of the last W prompt
 * positions before the first step.  Errors (nothing launched): length + 1 > C,
 * W > length, 0 < interval < W, n_delay < 0.  workspace >=
 * egs_latent_decode_workspace(shape) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t length;      /* entries in use (in / out) */
  int32_t generated;   /* tokens generated so far (in / out) */
  int32_t n_delay;     /* N_D: first compression after this many tokens */
  int32_t interval;    /* then every `interval` tokens; 0 = once; else >= n_obs */
  int32_t compressed;  /* out: 1 when this call compressed the cache */
} egs_latent_state;

size_t egs_latent_decode_workspace(const egs_decode_shape* shape);
egs_status egs_latent_decode_step(const egs_decode_shape* shape,
                                  const egs_retain_params* params,
                                  egs_latent_state* state, const void* q_new,
                                  const void* k_new, const void* v_new,
                                  void* q_window, void* k_cache, void* v_cache,
                                  void* out, int32_t* keep_idx, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Page-level retention ([EP] Sec. 7, GQA unions and physical page budgets):
 * whole pages of page_size consecutive cache entries are kept or released.
 *
 *   pages P_i = [i*S, (i+1)*S) clipped to [0, L), i < N_P = ceil(L / S)
 *   I_x(P_i) = max over t in P_i of token_scores[b, x, t]   (page importance)
 *   forced pages: every page holding a sink (t < n_sink) or a recent
 *                 position (t >= L - n_recent) of the decode shape
 *   K_x = forced pages U the n_keep_pages best other pages under
 *         (I_x descending, page index ascending)
 *   EGS_PAGE_GROUP:        set (b, g) = K_g      token_scores [B, Hkv, L]
 *                          (e.g. the group scores mu of egs_kv_retain)
 *   EGS_PAGE_HEAD_UNION:   set (b, g) = union over the heads h of group g of
 *                          K_h                   token_scores [B, Hq, L]
 *   EGS_PAGE_LAYER_UNION:  set (b, 0) = union over the groups g of K_g
 *                          (one physical block holds every group)
 *                          token_scores [B, Hkv, L]
 * Outputs: page_idx [B, Y, cap] int32 ascending, -1 past page_cnt[b, y];
 * page_cnt [B, Y] int32; Y = Hkv (GROUP, HEAD_UNION) or 1 (LAYER_UNION);
 * cap = egs_page_retain_capacity(...) = min(N_P, forced + m * n_keep_pages)
 * with m members per set (1, r or Hkv).  The decode shape's cache_len,
 * batch, head counts, n_sink and n_recent are used; its n_keep is not.
 * Valid: page_size >= 1, n_keep_pages >= 0, N_P <= 262144.  Capacity and
 * workspace queries return -1 / 0 for invalid arguments.
 * ------------------------------------------------------------------------- */
typedef enum {
  EGS_PAGE_GROUP = 0,
  EGS_PAGE_LAYER_UNION = 1,
  EGS_PAGE_HEAD_UNION = 2
} egs_page_mode;

int32_t egs_page_retain_capacity(const egs_decode_shape* shape, int32_t page_size,
                                 int32_t n_keep_pages, int32_t mode);
size_t egs_page_retain_workspace(const egs_decode_shape* shape, int32_t page_size,
                                 int32_t n_keep_pages, int32_t mode);
egs_status egs_page_retain(const egs_decode_shape* shape, int32_t page_size,
                           int32_t n_keep_pages, int32_t mode,
                           const float* token_scores, int32_t* page_idx,
                           int32_t* page_cnt, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Status helpers. */
const char* egs_status_string(egs_status status);
const char* egs_last_error(void);
int32_t egs_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EGS_H_ */
