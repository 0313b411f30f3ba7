/*
 * ckv.h -- C ABI of libckv.so: ClusterKV's clustering, recall and sparse
 * attention on one AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows (cited by title and section):
 *   "ClusterKV article": the intelliparadigm.com article
 *     "大模型KV Cache压缩技术：ClusterKV的语义空间优化", a write-up of the DAC'25
 *     paper "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
 *     Recallable Compression".
 *   "ClusterKV abstract": the arxivdaily.com listing of arXiv 2412.03213
 *     (recall at semantic-cluster granularity; clustering, selection,
 *     indexing and caching).
 *
 * Vocabulary.  A *unit* is one KV head of one sequence of one layer:
 * unit u = b * n_kv_heads + h.  Query head g of KV head h is query head
 * h * group + g (grouped-query attention).  head_dim must be 128.  Tokens
 * [0, n_sink) are sinks and never clustered; tokens [n_sink, n_clustered)
 * are clustered; tokens [n_clustered, n_total) are recent and not yet
 * clustered.  m = n_clustered - n_sink.
 *
 * Data types.  bf16 buffers are uint16_t bit patterns.  All pointers in
 * ckv_layer and all array arguments are DEVICE pointers (hipMalloc'd memory
 * of the current device), 16-byte aligned, owned by the caller.  The library
 * allocates and frees nothing, keeps no global state beyond a thread-local
 * error string, and never synchronises: every call enqueues work on the given
 * HIP stream (NULL = the legacy default stream) and returns; results are
 * valid once that stream has reached them.
 *
 * Errors.  Every entry point returns CKV_OK (0) or a negative code.  Argument
 * errors are detected on the host before anything is enqueued, so a failed
 * call writes nothing.  ckv_last_error() returns a thread-local text for the
 * last failing call on this thread.
 *
 * Calls that use the workspace take a caller-owned device buffer of at least
 * ckv_workspace_bytes() bytes.  The workspace must be zero-filled once before
 * its first use (ckv_workspace_init does that on the stream).  Calls sharing
 * one workspace must be ordered (same stream, or synchronised); calls on
 * different workspaces and different layers are independent.
 */
#ifndef CKV_H
#define CKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CKV_OK 0
#define CKV_EINVAL (-1)       /* null/misaligned pointer, size out of range   */
#define CKV_ENOSPACE (-2)     /* workspace too small, cache capacity exceeded */
#define CKV_EHIP (-3)         /* HIP launch or runtime error                  */
#define CKV_EUNSUPPORTED (-4) /* head_dim != 128, group > 16, K > 1024        */

#define CKV_HEAD_DIM 128
#define CKV_MAX_GROUP 16
#define CKV_MAX_CLUSTERS 1024

/* One layer's cache and cluster state (a plain struct the caller fills). */
typedef struct ckv_layer {
  int32_t batch;        /* sequences                                         */
  int32_t n_kv_heads;   /* KV heads per layer; units = batch * n_kv_heads    */
  int32_t group;        /* query heads per KV head, 1..16                    */
  int32_t head_dim;     /* must be 128                                       */
  int32_t n_sink;       /* unclustered leading tokens (16 in the method)     */
  int32_t n_clusters;   /* K, 1..1024                                        */
  int32_t capacity;     /* token rows per unit in k_tok / v_tok              */
  int32_t n_total;      /* tokens in the cache; the library advances it     */
  int32_t n_clustered;  /* sinks + clustered tokens; the library advances it */
  int32_t n_pending;    /* token count clustered by an uncommitted
                           ckv_cluster_incremental_async call, else 0; set to 0
                           initially, the library maintains it              */
  /* token-order cache, bf16 [units, capacity, 128] */
  uint16_t* k_tok;
  uint16_t* v_tok;
  /* cluster-ordered copy of the clustered rows, bf16 [units, capacity - n_sink, 128];
     row p holds token perm[p] */
  uint16_t* k_clu;
  uint16_t* v_clu;
  /* second copy of the same shape, written by ckv_cluster_incremental and
     then swapped with k_clu / v_clu (may be NULL if incremental is never used) */
  uint16_t* k_clu_alt;
  uint16_t* v_clu_alt;
  uint16_t* cdir;       /* bf16 [units, K, 128]: unit-direction centroids used for assignment */
  double* csum;         /* f64 [units, K, 128]: sum of members' unit keys                     */
  double* msum;         /* f64 [units, K, 128]: sum of members' keys                          */
  float* cmean;         /* f32 [units, K, 128]: mean key (scoring centroid); 0 if empty       */
  int32_t* csize;       /* [units, K]: members per cluster                                    */
  int32_t* offsets;     /* [units, K + 1]: cluster j = positions offsets[j] .. offsets[j+1]-1 */
  int32_t* assign;      /* [units, capacity - n_sink]: cluster of token n_sink + i            */
  int32_t* perm;        /* [units, capacity - n_sink]: token id at cluster-order position p   */
  /* second copies of offsets and cmean, written by ckv_cluster_incremental_async and
     swapped in by ckv_cluster_commit (may be NULL if the asynchronous form is never used) */
  int32_t* offsets_alt; /* [units, K + 1] */
  float* cmean_alt;     /* f32 [units, K, 128] */
} ckv_layer;

/* Text of the last error on this thread ("" if none).  Never NULL. */
const char* ckv_last_error(void);

/* sizeof(ckv_layer), so that language bindings can check their mirror of it. */
size_t ckv_abi_layer_bytes(void);

/* Bytes of workspace every call on layer L needs for budgets up to max_budget.
 * Returns 0 if L is invalid (see ckv_last_error). */
size_t ckv_workspace_bytes(const ckv_layer* L, int32_t max_budget);

/* Zero-fill a workspace on stream s (with a kernel, so it may be captured in a
 * HIP graph).  ws: device pointer, 16-byte aligned; ws_bytes > 0. */
int ckv_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Prefill clustering (ClusterKV article §3.2 prefill; §3.1 centroid; §4.1 layout).
 * Clusters tokens [n_sink, n) of every unit into K clusters by cosine K-means:
 *   init     c_j = bf16(x_I(j) / |x_I(j)|) where I are K distinct indices in
 *            [0, m), m = n - n_sink, into the clustered tokens: the draw
 *            ckv_init_indices makes from `seed` (the article does not say how
 *            K-means is initialised; the reading taken is a uniform draw
 *            without replacement);
 *   iters rounds of: a_i = argmax_j x_i . c_j (ties -> smallest j);
 *            S_j = sum of unit keys of members; c_j = bf16_rne(S_j / |S_j|)
 *            (empty or zero-sum clusters keep c_j);
 * then writes, from the final labels: assign, csize, offsets, perm (stable:
 * ascending token id inside a cluster), csum, msum, cmean = msum / csize,
 * and the cluster-ordered rows k_clu / v_clu.
 * Reads k_tok / v_tok rows [0, n).  Requires n_sink >= 0, 1 <= K <= m,
 * n <= capacity, iters >= 1, and no pending ckv_cluster_incremental_async
 * result.  Sets n_total = n_clustered = n on success.
 */
int ckv_cluster_prefill(ckv_layer* L, int32_t n, int32_t iters, uint64_t seed, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * The seeded initial indices of ckv_cluster_prefill (its initialisation
 * step, exposed so that callers can inspect or reuse the draw): for every
 * unit u, K distinct indices in [0, m), m = n - n_sink, drawn by Floyd's
 * sampling algorithm (Bentley and Floyd, CACM 1987) from the outputs of
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) started from state
 * seed + u: for j = m - K .. m - 1, t = r mod (j + 1) for the next output r;
 * t is taken unless already taken, else j.  init_idx[u, j] is the j-th index
 * taken (device int32 [units, K], written).  Requirements as for the prefill's
 * n; no workspace.
 */
int ckv_init_indices(const ckv_layer* L, int32_t n, uint64_t seed, int32_t* init_idx, void* stream);

/*
 * ckv_cluster_prefill from caller-given initial indices instead of a seed:
 * init_idx is device int32 [units, K], K distinct indices in [0, m) per unit;
 * an index outside [0, m) gives a zero direction: -1 holds slot j in reserve
 * for ckv_cluster_split (a zero direction scores 0 against every key, so the
 * slot stays empty unless a key scores below 0 against every other
 * direction).  Everything else as for ckv_cluster_prefill.
 */
int ckv_cluster_prefill_indices(ckv_layer* L, int32_t n, int32_t iters, const int32_t* init_idx, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * Append one decoded token per unit (ClusterKV article §3.2, decoding-stage
 * updates: every generated token's key and value join the cache; it stays
 * unclustered, and is attended as a recent row, until the next incremental
 * clustering pass takes it in).  k_new, v_new are bf16 [units, 128]
 * (device).  Writes row n_total of k_tok / v_tok and advances n_total.
 * CKV_ENOSPACE if n_total == capacity (nothing is written).
 */
int ckv_append(ckv_layer* L, const uint16_t* k_new, const uint16_t* v_new, void* stream);

/*
 * Incremental clustering (ClusterKV article §3.2 decoding-stage update): the
 * recent tokens [n_clustered, n_total) are assigned to the current directions
 * (ties -> smallest j), added to csum / msum / csize, and the touched
 * clusters get c_j = bf16_rne(csum_j / |csum_j|) (if nonzero) and
 * cmean_j = msum_j / csize_j.  Old tokens keep their cluster; K is unchanged.
 * The index (offsets, perm) is rebuilt over all clustered tokens and the
 * cluster-ordered copy is rewritten into k_clu_alt / v_clu_alt, which are then
 * swapped with k_clu / v_clu in *L.  The caller decides when to call it (the
 * method does so every 320 decoded tokens).  Requires the state written by a
 * previous prefill or incremental call (assign / csize / csum / msum of the
 * already clustered tokens), non-NULL k_clu_alt / v_clu_alt and no pending
 * ckv_cluster_incremental_async result.  A call with no recent tokens does
 * nothing.  Sets n_clustered = n_total.
 */
int ckv_cluster_incremental(ckv_layer* L, void* ws, size_t ws_bytes, void* stream);

/*
 * Asynchronous incremental clustering (ClusterKV article §4.1: clustering runs
 * beside decoding and its result is swapped in).  Computes exactly what
 * ckv_cluster_incremental computes for the recent tokens [n_clustered, n_total),
 * but leaves untouched every buffer that ckv_select, ckv_append_select and
 * ckv_sparse_decode read: the new index and scoring means go to offsets_alt and
 * cmean_alt, the new cluster-ordered copy to k_clu_alt / v_clu_alt.  The state
 * only clustering reads (csum, msum, csize, cdir, assign, perm) is updated in
 * place.  Records n_pending = n_total; nothing becomes current until
 * ckv_cluster_commit.
 * While the call's work runs on `stream`, recall, decode and appends may run on
 * another stream against the old state, with a different workspace: tokens
 * appended meanwhile are rows >= n_pending and stay recent.  No other
 * clustering call on the layer until the commit.
 * Requires non-NULL offsets_alt, cmean_alt, k_clu_alt, v_clu_alt and
 * n_pending == 0 (CKV_EINVAL otherwise).  With no recent tokens it enqueues
 * nothing and leaves n_pending at 0.
 */
int ckv_cluster_incremental_async(ckv_layer* L, void* ws, size_t ws_bytes, void* stream);

/*
 * Make the last ckv_cluster_incremental_async result current (host only,
 * enqueues nothing): swaps offsets / offsets_alt, cmean / cmean_alt,
 * k_clu / k_clu_alt and v_clu / v_clu_alt in *L, sets n_clustered = n_pending
 * and n_pending = 0.  The caller orders every later call that reads the layer
 * after the async call's work (an event recorded on its stream, waited on by
 * the other stream).  CKV_EINVAL if nothing is pending.
 */
int ckv_cluster_commit(ckv_layer* L);

/*
 * The assignment step alone (ClusterKV article §3.2 prefill, cosine K-means;
 * §4.1 half-precision distance computation): for the tokens [n_sink, n) of
 * every unit, a_i = argmax_j k_i . cdir_j (ties -> smallest j), written to
 * assign[u, 0 : n - n_sink].  It is the first step of every Lloyd round of
 * ckv_cluster_prefill (bf16 MFMA distances with the argmax fused, scores never
 * stored), exported so that callers can run or time it on its own.  Reads
 * k_tok rows [n_sink, n) and cdir; writes only assign, so csize, offsets,
 * perm, the sums and the cluster-ordered rows no longer describe the labels
 * until the next ckv_cluster_prefill.  Requires n_sink < n <= capacity and
 * no pending ckv_cluster_incremental_async result; no workspace.
 */
int ckv_assign(const ckv_layer* L, int32_t n, void* stream);

/*
 * Drift-triggered split (ClusterKV article §3.2, decoding-stage updates: a
 * cluster whose mean intra-cluster distance passes a threshold is split).
 * Per unit, over the clustered tokens [n_sink, n_clustered):
 *   drift_j  = 1 - |csum_j| / csize_j, the mean cosine distance of the members
 *              to the centre direction csum_j / |csum_j| (in [0, 1]);
 *   pairs    clusters with csize_j >= 2 and drift_j > threshold, in decreasing
 *              drift (ties -> smaller j), are paired with the empty slots
 *              (csize_f == 0) in increasing f, as far as the empty slots go;
 *   split    the member of j with the smallest cosine to c_j (ties -> earliest
 *              token) gives c_f = bf16_rne(x / |x|); each member of j moves to
 *              f when x . c_f > x . c_j (>= when f < j).
 * These dot products and cosines are f64 over the bf16 values.  Then, as after
 * the last prefill round, assign, csize, offsets, perm, csum, msum, cmean, cdir
 * (nonempty clusters; an empty one keeps its direction) and k_clu / v_clu are
 * rewritten in place from the labels of all clustered tokens.  Clusters no
 * split touched keep their members; their sums are added again in another
 * order and may change in the last bits.
 * Empty slots come from prefill (init_idx -1) or from clusters K-means left
 * empty; without one nothing splits.  The caller picks threshold (any non-NaN
 * value) and when to call (e.g. after each incremental pass).  Requires the
 * state of a prefill or incremental call and n_pending == 0 (CKV_EINVAL
 * otherwise); no other call on the layer may run meanwhile on another stream.
 * n_total and n_clustered are unchanged.
 */
int ckv_cluster_split(ckv_layer* L, double threshold, void* ws, size_t ws_bytes, void* stream);

/*
 * Cluster-granularity recall (ClusterKV article §3.3; GQA reading: one recall
 * per KV head with the group's summed query q_bar = sum_g q_g).
 *   q:        bf16 [batch, n_kv_heads * group, 128] (device)
 *   sel_pos:  int32 [units, budget] (device, written): ascending cluster-order
 *             positions of the recalled tokens in the first sel_count[u] slots
 *   sel_count int32 [units] (device, written): exactly min(budget, m)
 * Clusters are visited by descending q_bar . cmean_j (ties -> smaller j; empty
 * clusters never), taken whole while they fit in the remaining budget; the
 * first cluster that does not fit contributes its highest-q_bar.k tokens
 * (ties -> smaller position) to fill the budget exactly.  Requires
 * n_clustered - n_sink >= K, budget >= 0.
 */
int ckv_select(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
               int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/*
 * ckv_append followed by ckv_select in one launch (one decode step's token
 * write and recall): writes k_new / v_new (bf16 [units, 128], device) into
 * row n_total of k_tok / v_tok, recalls exactly as ckv_select does (recall
 * never reads the token-order rows), and advances n_total.  Errors as for
 * either call; nothing is enqueued on error.
 */
int ckv_append_select(ckv_layer* L, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                      int32_t budget, int32_t* sel_pos, int32_t* sel_count, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Per-query-head recall (ClusterKV article §3.3 recall stated for a single
 * query, applied to each query head separately; the other reading of
 * grouped-query attention, where the G heads of a KV head do not share one
 * set).  Exactly ckv_select with G = 1 for every query head:
 *   sel_pos   int32 [units * group, budget] (device, written): set s = u * group + g
 *             is the recall of query head g of unit u, scored with q_g alone
 *   sel_count int32 [units * group] (device, written): min(budget, m)
 * The workspace must hold ckv_workspace_bytes_per_head() bytes.  Errors as
 * for ckv_select.
 */
size_t ckv_workspace_bytes_per_head(const ckv_layer* L, int32_t max_budget);
int ckv_select_per_head(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                        int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse decode with one recalled set per query head (the output of
 * ckv_select_per_head): out[b, h * group + g, :] attends to the sinks, the
 * sel_count[s] rows listed in sel_pos[s, :] (s = u * group + g, row stride
 * `budget`) and the recent rows.  Layouts, limits and errors as for
 * ckv_sparse_decode; the workspace must hold ckv_workspace_bytes_per_head()
 * bytes, and its first 4 * units * group bytes are arrival counters left zero.
 */
int ckv_sparse_decode_per_head(const ckv_layer* L, const uint16_t* q, const int32_t* sel_pos,
                               const int32_t* sel_count, int32_t budget, float* out, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * Sparse decode (ClusterKV article §3.1 attention; §4.1 cluster-contiguous
 * rows): for every query head g of unit u,
 *   out[b, h * group + g, :] = softmax(q_g . K_S^T / sqrt(128)) V_S
 * over S = sinks [0, n_sink) of k_tok/v_tok, the sel_count[u] rows of
 * k_clu/v_clu listed in sel_pos[u, :] (row stride `budget`), and the recent
 * rows [n_clustered, n_total) of k_tok/v_tok.  out is f32
 * [batch, n_kv_heads * group, 128] (device, written); an empty S gives 0.
 * sel_count[u] must be <= min(budget, m) and every listed position < m.
 * The first 4 * units bytes of the workspace are per-unit arrival counters of
 * the split-K merge; a call leaves them zero, as ckv_workspace_init does.  The
 * workspace starts with 8 * units * group bytes of such counters for every call
 * (both recall modes); clustering calls never write them.
 */
int ckv_sparse_decode(const ckv_layer* L, const uint16_t* q, const int32_t* sel_pos,
                      const int32_t* sel_count, int32_t budget, float* out, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * Recall and sparse decode of one decode step in a single launch (ClusterKV
 * article §3.3 selection procedure, §3.1 attention over the recalled tokens,
 * §4.1 cluster-contiguous rows).  Computes exactly what ckv_select followed by
 * ckv_sparse_decode computes:
 *   sel_pos   int32 [units, budget] (device, written): the recalled
 *             cluster-order positions, ascending, in the first sel_count[u]
 *             slots -- the same positions ckv_select writes;
 *   sel_count int32 [units] (device, written): min(budget, m);
 *   out       f32 [batch, n_kv_heads * group, 128] (device, written): every
 *             query head's attention over the sinks, the recalled rows and the
 *             recent rows [n_clustered, n_total).
 * The recalled positions are not read back: each of the set's workgroups
 * recalls the set itself and streams its share of the rows straight from the
 * index, so no hand-off between a recall launch and a decode launch sits
 * between the query and the output.  The decode's floating-point sums run in
 * another order than ckv_sparse_decode's, so out may differ from it in the
 * last bits.  Requirements and errors as for ckv_select and
 * ckv_sparse_decode; the workspace holds ckv_workspace_bytes() bytes and its
 * arrival counters are left zero.
 *   next      a layer whose call follows this one on the stream (the next
 *             layer of the model), or NULL: a hint only.  When it has the same
 *             batch, n_kv_heads and n_clusters as L, the workgroups that finish
 *             early read its cmean and offsets into the device caches, so that
 *             its own call starts from cached centroids.  Nothing of *next is
 *             written; results never depend on it.
 */
int ckv_select_decode(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                      int32_t* sel_count, float* out, const ckv_layer* next, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * ckv_append, then ckv_select_decode, in one launch (one decode step of one
 * layer): k_new / v_new (bf16 [units, 128], device) become row n_total of
 * k_tok / v_tok and are attended as the newest recent row; n_total advances.
 * Errors as for either call; nothing is enqueued on error.
 */
int ckv_append_select_decode(ckv_layer* L, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                             int32_t budget, int32_t* sel_pos, int32_t* sel_count, float* out, const ckv_layer* next,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * ckv_select_per_head followed by ckv_sparse_decode_per_head in one launch
 * (ClusterKV article §3.3 applied to every query head): sel_pos int32
 * [units * group, budget], sel_count int32 [units * group], out as for
 * ckv_sparse_decode, next as for ckv_select_decode.  The workspace must hold
 * ckv_workspace_bytes_per_head() bytes.
 */
int ckv_select_decode_per_head(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                               int32_t* sel_count, float* out, const ckv_layer* next, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * ckv_select_decode for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Computes
 * exactly what ckv_select_decode computes (the same kernel, the same bits),
 * with no workspace argument: its scratch (arrival counters, split-K
 * partials, cut-cluster scores) is a file-scope device array of
 * ckv_select_decode_noalloc_limit() bytes (16 MiB) that each GPU holds from
 * the library's first such call on it until the process ends.  The call
 * allocates and frees nothing.  The first call on a device zero-fills the
 * counters with a kernel on `stream`; every call leaves them zero.  Needs
 * 64 KiB + units * W * 4 * tier(group) * 130 + units * (capacity - n_sink) * 4
 * bytes (W <= 64 chunks per unit, tier = group rounded up to a power of two);
 * a larger layer returns CKV_ENOSPACE before anything is enqueued.  All calls
 * on one GPU share the array: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race and give wrong results.
 * Other errors as for ckv_select_decode.
 */
size_t ckv_select_decode_noalloc_limit(void);
int ckv_select_decode_noalloc(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                              int32_t* sel_count, float* out, const ckv_layer* next, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CKV_H */
