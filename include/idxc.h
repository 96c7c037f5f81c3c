/*
 * idxc.h — C ABI of libidxc.so: the IndexCache hot path on AMD MI355X (gfx950).
 *
 * What the library computes (sources are web pages, cited by title + section):
 *
 *  [W] "IndexCache：跨层复用稀疏注意力的索引" (wineandchord.com), section
 *      "从 DSA 的成本分解开始" (starting from DSA's cost decomposition): each
 *      layer has a role c_l in {F, S}; an F layer runs its own indexer and
 *      produces I_l = TopK(s_l, k), overwriting the cache; an S layer runs no
 *      indexer and uses the latest F layer's index tensor; the first layer
 *      must be F. Its executable state machine raises an error for a wrong
 *      length, a first role other than F, or a role outside {F, S}.
 *  [J] "NLP——IndexCache" notes (joezjh.github.io), section "IndexCache 方法":
 *      T_t^(l) <- T_t^(f(l)), f(l) = max{j < l : c_j = F}; in the layer loop,
 *      F computes and caches the indices, S reads the cache. Section
 *      "背景 & 问题提出": a lightning indexer picks, for every query, the top-k
 *      (k = 2048) of all previous tokens; core attention then runs on those k.
 *
 *  Where the pages name an operation but do not define it, this library uses:
 *   - indexer score  s[t, s'] = sum_h w[t,h] * max(0, q_I[t,h,:] . k_I[s',:]),
 *     one indexer key per token shared by all indexer heads, candidates
 *     s' in [0, t] (the query's own position included);
 *   - top-k order: higher score first, then lower position, -0.0 == +0.0;
 *     output sorted in that order, min(k, t+1) entries, then -1 padding;
 *   - core attention O[t,h] = sum_{s in I_t} softmax(scale * Q[t,h].K[s]) V[s]
 *     over the valid (non -1) entries, one shared K/V head (MQA).
 *
 * Conventions shared by every entry point
 *  - All tensors are row-major and contiguous, in DEVICE memory owned by the
 *    caller. The library never allocates, frees or keeps a tensor, and keeps
 *    no state between calls. Every device pointer must be 16-byte aligned.
 *  - Layouts (bf16 = IEEE bfloat16 stored as uint16):
 *      q_idx   [B, Lq, H_I, d_I] bf16     k_idx [B, Lk, d_I] bf16
 *      w       [B, Lq, H_I]      bf16
 *      q       [B, Lq, H, D]     bf16     k, v  [B, Lk, D]   bf16
 *      out     [B, Lq, H, D]     bf16
 *      scores  [B, Lq, Lk]       fp32     indices [B, Lq, k] int32
 *    Query row i of batch b sits at absolute position t = q_pos0 + i and may
 *    attend to keys 0..t of the same batch; q_pos0 + Lq <= Lk is required
 *    (prefill: q_pos0 = 0, Lq = Lk; decode: Lq = 1, q_pos0 = Lk - 1; a query
 *    chunk c of size C: q_pos0 = c*C, Lk = (c+1)*C).
 *  - Supported sizes: d_I in {32, 64, 128}; 1 <= H_I <= 64; D in {64, 128};
 *    1 <= H <= 64; 1 <= k <= 2048; Lk <= 2^24; B*Lq <= 2^24. Anything else
 *    returns IDXC_ERR_UNSUPPORTED.
 *  - Calls are asynchronous on the given HIP stream (NULL = the default
 *    stream). The returned status covers argument checks and launch errors;
 *    a fault inside a kernel surfaces at the caller's next synchronisation.
 *    All argument checks run on the host before any launch, so a call that
 *    returns an error has launched nothing and touched no device memory.
 *  - Thread safety: calls on distinct streams with distinct buffers may run
 *    concurrently. The error message is thread-local.
 *  - NaN or infinite inputs are outside the contract.
 */
#ifndef IDXC_H
#define IDXC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IDXC_OK = 0,
  IDXC_ERR_INVALID_ARG = 1, /* null pointer, misaligned pointer, size < 1,
                               q_pos0 + Lq > Lk, workspace too small */
  IDXC_ERR_PATTERN = 2,     /* pattern length != n_layers, role not in {F,S},
                               first role not F */
  IDXC_ERR_UNSUPPORTED = 3, /* sizes outside the compiled set (see above) */
  IDXC_ERR_HIP = 4          /* HIP runtime error at launch */
} idxc_status;

/* Problem sizes. q_pos0 = absolute position of query row 0. */
typedef struct {
  int32_t B, Lq, Lk, q_pos0;
  int32_t H_I, d_I; /* indexer heads, indexer head dim */
  int32_t H, D;     /* attention query heads, head dim (one shared KV head) */
  int32_t k;        /* top-k size */
} idxc_dims;

/* Per-layer device pointers for idxc_layer_stack_forward. q_idx, k_idx and w
 * are read on F layers only and may be NULL on S layers. */
typedef struct {
  const void* q_idx;
  const void* k_idx;
  const void* w;
  const void* q;
  const void* k;
  const void* v;
  void* out;
} idxc_layer;

/* Message describing the last non-OK status returned on this thread ("" if
 * none). The pointer stays valid until the next idxc call on this thread. */
const char* idxc_last_error(void);

/* Library version string, e.g. "idxc 0.1.0 gfx950". */
const char* idxc_version(void);

/* Host-only pattern check: [W] state machine rules. Writes the number of F
 * layers to *n_full (may be NULL). No device is touched. */
int idxc_validate_pattern(const char* pattern, int32_t n_layers, int32_t* n_full);

/* Host-only nearest-F map: source[l] = l if c_l = F, else
 * f(l) = max{j < l : c_j = F} ([J] "IndexCache 方法"). source has n_layers
 * int32 entries in HOST memory. No device is touched. */
int idxc_schedule(const char* pattern, int32_t n_layers, int32_t* source);

/* Lightning-indexer scores, materialised ([J] "背景 & 问题提出": the indexer
 * scores every query against all earlier tokens). Writes scores[b,i,s] for
 * every s in [0, Lk): the fp32 score for s <= t, -inf for s > t; -0.0 is
 * written as +0.0. Reads q_idx, k_idx, w. Uses B, Lq, Lk, q_pos0, H_I, d_I.
 * MFMA bf16 products with fp32 accumulation: on integer-valued inputs whose
 * sums stay below 2^24 the result is exact. */
int idxc_indexer_scores(const void* q_idx, const void* k_idx, const void* w,
                        const idxc_dims* dims, float* scores, void* hip_stream);

/* Order of the positions in an output index list. The selected set is the
 * same in both: the min(k, t+1) best positions under (score desc, position
 * asc), followed by -1 entries.
 *   IDXC_ORDER_SCORE:    sorted by (score desc, position asc);
 *   IDXC_ORDER_POSITION: increasing position (what a layer stack's index
 *                        cache holds; attention does not depend on order). */
enum { IDXC_ORDER_SCORE = 0, IDXC_ORDER_POSITION = 1 };

/* Per-query top-k of materialised scores ([W] I_l = TopK(s_l, k)). Row (b,i)
 * reads scores[b,i,0..t] only (t = q_pos0 + i) and writes indices[b,i,0..k-1]:
 * the min(k, t+1) best positions in the given order (IDXC_ORDER_*, anything
 * else is IDXC_ERR_INVALID_ARG), then -1. Uses B, Lq, Lk, q_pos0, k.
 * Bit-exact and deterministic. With Lk <= 65536 this is one launch and
 * needs no workspace; longer rows are selected in three launches through a
 * device workspace of at least idxc_topk_workspace_bytes() bytes (per-chunk
 * histograms and a per-row candidate list; NULL/0 is fine when that is 0);
 * any Lk up to 2^24 is supported. */
int idxc_topk(const float* scores, const idxc_dims* dims, int32_t order, void* workspace,
              size_t workspace_bytes, int32_t* indices, void* hip_stream);

/* Workspace bytes idxc_topk needs for these sizes: 0 when Lk <= 65536, else
 * B * Lq * (ceil(Lk / 8192) * 4096 + 16384 * 8 + 4). Host-only. */
int idxc_topk_workspace_bytes(const idxc_dims* dims, size_t* bytes);

/* Bytes of device workspace for these sizes (written to *bytes), host-only:
 * with dims->H and dims->D set (> 0), what idxc_layer_stack_forward needs at
 * full speed; with H = D = 0, what idxc_indexer_topk needs at full speed. */
int idxc_workspace_bytes(const idxc_dims* dims, size_t* bytes);

/* Fused indexer + top-k: same result as idxc_indexer_scores followed by
 * idxc_topk with the same order, without writing the score matrix. Scores are filtered on chip
 * against a running per-query threshold; only candidates that can still be
 * in the top-k are kept, in a caller-provided workspace. Smaller workspaces
 * (down to 256*ceil(4*B*Lq/256) + 8*B*Lq*64*ceil((k+64)/64) bytes) are
 * accepted and only cost speed.
 * Returns IDXC_ERR_INVALID_ARG if the workspace is smaller than that. */
int idxc_indexer_topk(const void* q_idx, const void* k_idx, const void* w,
                      const idxc_dims* dims, int32_t order, void* workspace,
                      size_t workspace_bytes, int32_t* indices, void* hip_stream);

/* Gathered sparse attention ([J] "背景 & 问题提出": core attention only over
 * the k selected tokens). For each (b,i,h): softmax over the valid entries of
 * indices[b,i,:] (entries equal to -1 are skipped; every other entry must be
 * in [0, Lk)) of scale * q[b,i,h,:] . k[b,s,:], then the weighted sum of
 * v[b,s,:], written to out[b,i,h,:] as bf16. A row with no valid entry gets
 * zeros. Uses B, Lq, Lk, H, D, k. fp32 softmax and accumulation, bf16 P.
 * scale must be finite and > 0 (a NaN, infinite, zero or negative scale is
 * IDXC_ERR_INVALID_ARG).
 * workspace (optional, NULL = none): with at least
 * idxc_sparse_attn_workspace_bytes() bytes, calls with few query rows split
 * each index list over several workgroups and merge the partial results. */
int idxc_sparse_attn(const void* q, const void* k, const void* v,
                     const int32_t* indices, const idxc_dims* dims, float scale,
                     void* workspace, size_t workspace_bytes, void* out,
                     void* hip_stream);

/* Workspace bytes that let idxc_sparse_attn split index lists (0 when it
 * would not split for these sizes). Host-only. */
int idxc_sparse_attn_workspace_bytes(const idxc_dims* dims, size_t* bytes);

/* The whole hot path over a stack of n_layers layers ([W] state machine,
 * [J] layer loop). The pattern (n_layers chars in {F,S}, first F) is checked
 * before anything runs. For each layer l in order: if F, the fused indexer +
 * top-k of layers[l] overwrites index_cache [B,Lq,k] and *indexer_calls is
 * incremented; then sparse attention of layers[l] reads index_cache and
 * writes layers[l].out. S layers launch no indexer work. Afterwards
 * index_cache holds the last F layer's indices, in IDXC_ORDER_POSITION
 * (attention does not depend on the order, and position order lets the K/V
 * gathers of the rows that run together sweep the keys together).
 * *indexer_calls (HOST
 * pointer) receives the number of indexer launches (= number of F layers).
 * debug_indices, if not NULL, is a DEVICE buffer [n_layers, B, Lq, k] that
 * receives each layer's cache contents (for tests). workspace as for
 * idxc_indexer_topk, plus room for attention partials; idxc_workspace_bytes
 * with H and D set gives the full-speed size. scale as for idxc_sparse_attn
 * (finite and > 0). */
int idxc_layer_stack_forward(const char* pattern, int32_t n_layers,
                             const idxc_layer* layers, const idxc_dims* dims,
                             float scale, int32_t* index_cache, void* workspace,
                             size_t workspace_bytes, int32_t* indexer_calls,
                             int32_t* debug_indices, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * stack as idxc_layer_stack_forward, same arguments, results and checks, but
 * with no workspace argument. Its scratch (candidate lists, per-chunk top-k
 * segments, attention partials) is a library-owned device array of
 * IDXC_NOALLOC_SCRATCH_BYTES bytes per GPU, which each GPU the library runs
 * on holds from the first call until the process ends. The call uses the
 * array of the CURRENT device (hipGetDevice), so hip_stream must belong to
 * that device. Nothing is allocated or freed, by the library or by any
 * routine it calls.
 *  - Sizes whose minimum workspace (what idxc_workspace_bytes reports at its
 *    smallest, see idxc_indexer_topk) exceeds the array return
 *    IDXC_ERR_UNSUPPORTED before anything runs. Decode batches (for instance
 *    64 sequences of up to 196608 cached tokens at k = 2048) and short
 *    prefills fit; a 32768-token prefill does not.
 *  - Every call on one GPU shares that GPU's array: calls that overlap in time
 *    on one GPU (on different streams or from different threads) race and
 *    corrupt each other's results; serialise them. The array keeps the last
 *    call's contents; no result depends on them.
 *  - The first call on a device looks up the array's device address
 *    (hipGetSymbolAddress) and may initialise the HIP runtime; make it before
 *    a graph capture begins if the capture must see no runtime set-up. */
#define IDXC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int idxc_layer_stack_forward_noalloc(const char* pattern, int32_t n_layers,
                                     const idxc_layer* layers, const idxc_dims* dims,
                                     float scale, int32_t* index_cache, int32_t* indexer_calls,
                                     int32_t* debug_indices, void* hip_stream);

/* Ragged batches (per-sequence lengths and positions, as a serving batch
 * has them): like idxc_indexer_topk / idxc_layer_stack_forward, but query row
 * r = b*Lq + i sits at the absolute position q_pos[r] (DEVICE int32 [B*Lq])
 * instead of q_pos0 + i, and scores keys 0..q_pos[r] of its batch. Keys stay
 * in [B, Lk, d] buffers padded to the longest sequence (Lk); a row with
 * q_pos[r] < 0 selects nothing (all -1; its attention output is 0), and a
 * position >= Lk is read as Lk - 1. dims->q_pos0 is not used for positions
 * but must still pass the usual checks (0 is fine). A decode batch of
 * sequences with lengths n_b is B rows with Lq = 1, q_pos[b] = n_b - 1 and
 * Lk = max n_b. Workspace as for the uniform calls with the same dims. */
int idxc_indexer_topk_ragged(const void* q_idx, const void* k_idx, const void* w,
                             const idxc_dims* dims, const int32_t* q_pos, int32_t order,
                             void* workspace, size_t workspace_bytes, int32_t* indices,
                             void* hip_stream);
int idxc_layer_stack_forward_ragged(const char* pattern, int32_t n_layers,
                                    const idxc_layer* layers, const idxc_dims* dims,
                                    const int32_t* q_pos, float scale, int32_t* index_cache,
                                    void* workspace, size_t workspace_bytes,
                                    int32_t* indexer_calls, int32_t* debug_indices,
                                    void* hip_stream);

/* Multi-layer distillation loss of an index-sharing layer group ("NLP——
 * IndexCache" notes, section "方法二：Training-Aware IndexCache": the F layer's
 * indexer fits the attention distributions of every layer it serves;
 * Proposition 1 there: the gradient equals that of one KL against the mean
 * teacher). For query row r = (b, i) at t = q_pos0 + i, over keys 0..t:
 *   q = Softmax(logits[b,i,0..t]),
 *   row_loss[r] = (1/n) sum_j sum_s p_j[s] log(p_j[s] / q[s])   (0 log 0 = 0),
 *   grad[b,i,s] = q[s] - (1/n) sum_j p_j[s] for s <= t, 0 for s > t,
 * with p_j = teachers[j, b, i, :] (n = n_teachers distributions, each summing
 * to 1 over 0..t; entries past t are not read) and grad = d row_loss /
 * d logits. logits [B,Lq,Lk] fp32 (e.g. idxc_indexer_scores' output),
 * teachers [n_teachers,B,Lq,Lk] fp32, row_loss [B*Lq] fp32 and grad
 * [B,Lq,Lk] fp32, all DEVICE; row_loss or grad may be NULL. Uses B, Lq, Lk,
 * q_pos0. 1 <= n_teachers <= 64. fp32 arithmetic, deterministic.
 * Asynchronous on hip_stream. */
int idxc_distill_loss(const float* logits, const float* teachers, int32_t n_teachers,
                      const idxc_dims* dims, float* row_loss, float* grad, void* hip_stream);

/* Cross-layer agreement of two index tensors a, b [B,Lq,k] int32 (DEVICE;
 * entries are positions in [0, Lk) or -1, in any order; other values are
 * ignored). Per row, over the valid entries taken as sets: inter = |A ∩ B|,
 * overlap = |A ∩ B| / |A| (1 if both sets are empty, 0 if only A is) and
 * jaccard = |A ∩ B| / |A ∪ B| (1 if both are empty), the measures
 * "IndexCache：跨层复用稀疏注意力的索引" uses for how much adjacent layers'
 * top-k selections agree (with |A| = k, overlap = |A ∩ B| / k). Outputs are
 * DEVICE buffers of B*Lq entries; any may be NULL. Uses B, Lq, Lk, k.
 * Lk above 262144 returns IDXC_ERR_UNSUPPORTED (two bitmaps of Lk bits live
 * in LDS). Asynchronous on hip_stream. */
int idxc_overlap(const int32_t* a, const int32_t* b, const idxc_dims* dims, int32_t* inter,
                 float* overlap, float* jaccard, void* hip_stream);

/* Overlap matrix of n_layers index tensors sel [n_layers, B, Lq, k] int32
 * (DEVICE; for instance the debug_indices of an all-F idxc_layer_stack_forward,
 * i.e. every layer's own top-k): matrix[a * n_layers + b] = mean over the B*Lq
 * rows of overlap(sel[a], sel[b]) = |A ∩ B| / |A|, with the per-row
 * conventions of idxc_overlap (so the diagonal is 1). This is the adjacent-
 * and cross-layer agreement of "IndexCache：跨层复用稀疏注意力的索引",
 * section "相邻层重叠很高，但“重叠率”不是搜索目标" (Overlap equation), for
 * every pair of layers at once. matrix: DEVICE float [n_layers * n_layers].
 * workspace: DEVICE, 16-byte aligned, at least
 * idxc_overlap_matrix_workspace_bytes(n_layers) bytes; its contents on entry
 * do not matter. Deterministic (per-row ratios are summed as 32.32 fixed-point
 * integers; error below 2^-32 per row). n_layers above 64 or Lk above 262144
 * returns IDXC_ERR_UNSUPPORTED. Uses B, Lq, Lk, k. Asynchronous on hip_stream. */
size_t idxc_overlap_matrix_workspace_bytes(int32_t n_layers); /* 0 if n_layers is outside [1, 64] */
int idxc_overlap_matrix(const int32_t* sel, int32_t n_layers, const idxc_dims* dims,
                        void* workspace, size_t workspace_bytes, float* matrix,
                        void* hip_stream);

/* Loss callback of idxc_greedy_pattern: pattern is a NUL-terminated string of
 * n_layers roles ('F'/'S', first 'F'); returns the loss of running the model
 * with that pattern (lower is better). Called on the calling host thread. */
typedef double (*idxc_loss_fn)(const char* pattern, void* user);

/* Greedy F/S pattern search, host only ("IndexCache：跨层复用稀疏注意力的索引",
 * section "Training-free：直接用语言模型损失选择 Full 层"; "NLP——IndexCache"
 * notes, section "核心算法：Greedy Layer Selection"): start from all F with
 * layer 0 pinned to F; `removals` times, try every remaining F layer l >= 1 as
 * S, evaluate loss(trial pattern, user), and commit the lowest (ties go to the
 * lower layer). pattern: HOST buffer of n_layers + 1 chars, receives the
 * result. *evals (HOST, may be NULL) receives the number of loss calls,
 * sum_{i < removals} (n_layers - 1 - i). removals outside [0, n_layers - 1]
 * is IDXC_ERR_INVALID_ARG; a NaN loss stops the search with
 * IDXC_ERR_INVALID_ARG. No device is touched. */
int idxc_greedy_pattern(int32_t n_layers, int32_t removals, idxc_loss_fn loss, void* user,
                        char* pattern, int64_t* evals);

/* An overlap proxy loss for idxc_greedy_pattern when no model is at hand (the
 * pages drive the search with the language-model loss; this stand-in only
 * measures how much of each S layer's own selection its reused cache keeps):
 * loss = (1 / n_layers) * sum over S layers l of (1 - matrix[l][f(l)]), with
 * f(l) the latest F layer before l and matrix the HOST copy of an
 * idxc_overlap_matrix result [n_layers * n_layers]. Host only. */
int idxc_overlap_proxy_loss(const char* pattern, int32_t n_layers, const float* matrix,
                            double* loss);

#ifdef __cplusplus
}
#endif

#endif /* IDXC_H */
