// C ABI of libckv.so: host-side validation, workspace layout and launch
// orchestration.  Declarations and the full contract live in include/ckv.h.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/ckv.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CKV_OK;
  return fail(CKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t counters;  // [2 units] u32 arrival counters: decode, then select; zero between calls
  size_t aux;       // prefill: [units, K] int32 drawn indices; split: [units, 2K + 1] int32 pair plan
  size_t invn;      // prefill / incremental: [units, clu_cap] f64 inverse key norms
  size_t labs;      // prefill: [2, units, stride16] uint16 labels of alternate Lloyd rounds
  size_t scores;    // select: [units, K] f32
  size_t cut;       // select: [units, clu_cap] u32 keys of the cut cluster
  size_t partials;  // decode: [units, kMaxChunks, GT, 130] f32
  size_t total;
  size_t off_aux, off_invn, off_labs, off_scores, off_cut, off_partials;
  size_t off_rd_cut;  // fused recall + decode: cut scores after the partials
};

int group_tier(int g) {
  int t = 1;
  while (t < g) t <<= 1;
  return t;
}

// Row stride of the prefill's 16-bit label buffers: the clustered capacity
// rounded up to even, so rows and their dword loads stay aligned.
int label16_stride(const ckv_layer* L) { return (L->capacity - L->n_sink + 1) & ~1; }

// per_head: one recall / attention set per query head (units * group of them)
// instead of one per KV head.
Layout layout_of(const ckv_layer* L, bool per_head = false) {
  const size_t units = (size_t)L->batch * L->n_kv_heads;
  const size_t sets = units * (per_head ? (size_t)L->group : 1);
  const size_t clu_cap = (size_t)(L->capacity - L->n_sink);
  Layout w;
  // Arrival counters of both recall modes (decode at [0, sets), recall at
  // [sets, 2 sets)), sized for the per-query-head count whatever the mode, so
  // that the bodies below never overlap the counters of either mode when calls
  // of both modes share one workspace.
  w.counters = align256(units * (size_t)L->group * 2 * sizeof(uint32_t));
  w.aux = align256(units * (2 * (size_t)L->n_clusters + 1) * sizeof(int32_t));
  w.invn = align256(units * clu_cap * sizeof(double));
  w.labs = align256(2 * units * label16_stride(L) * sizeof(uint16_t));
  w.scores = align256(sets * L->n_clusters * sizeof(float));
  w.cut = align256(sets * clu_cap * sizeof(uint32_t));
  w.partials = align256(units * ckv::kMaxChunks * group_tier(L->group) * ckv::kPartialStride * sizeof(float));
  w.off_aux = w.counters;
  w.off_invn = w.counters + w.aux;
  w.off_labs = w.off_invn + w.invn;
  w.off_scores = w.counters;
  w.off_cut = w.counters + w.scores;
  w.off_partials = w.counters;
  w.off_rd_cut = w.counters + w.partials;
  size_t body = w.aux + w.invn + w.labs;
  if (w.scores + w.cut > body) body = w.scores + w.cut;
  if (w.partials + w.cut > body) body = w.partials + w.cut;
  w.total = w.counters + body;
  return w;
}

// Checks shared by every call that takes a layer.
int check_layer(const ckv_layer* L) {
  if (!L) return fail(CKV_EINVAL, "layer is NULL");
  if (L->head_dim != CKV_HEAD_DIM) return fail(CKV_EUNSUPPORTED, "head_dim %d != 128", L->head_dim);
  if (L->group < 1) return fail(CKV_EINVAL, "group %d < 1", L->group);
  if (L->group > CKV_MAX_GROUP) return fail(CKV_EUNSUPPORTED, "group %d > %d", L->group, CKV_MAX_GROUP);
  if (L->batch < 1 || L->n_kv_heads < 1) return fail(CKV_EINVAL, "batch and n_kv_heads must be >= 1");
  if ((long long)L->batch * L->n_kv_heads > (1 << 24)) return fail(CKV_EINVAL, "too many units");
  if (L->n_clusters < 1) return fail(CKV_EINVAL, "n_clusters %d < 1", L->n_clusters);
  if (L->n_clusters > CKV_MAX_CLUSTERS)
    return fail(CKV_EUNSUPPORTED, "n_clusters %d > %d", L->n_clusters, CKV_MAX_CLUSTERS);
  if (L->n_sink < 0) return fail(CKV_EINVAL, "n_sink %d < 0", L->n_sink);
  if (L->capacity <= L->n_sink) return fail(CKV_EINVAL, "capacity %d <= n_sink %d", L->capacity, L->n_sink);
  if (L->capacity > (1 << 30)) return fail(CKV_EINVAL, "capacity too large");
  if (L->n_total < 0 || L->n_total > L->capacity)
    return fail(CKV_EINVAL, "n_total %d outside [0, capacity]", L->n_total);
  if (L->n_clustered < 0 || L->n_clustered > L->n_total)
    return fail(CKV_EINVAL, "n_clustered %d outside [0, n_total]", L->n_clustered);
  if (L->n_pending != 0 && (L->n_pending < L->n_clustered || L->n_pending > L->n_total))
    return fail(CKV_EINVAL, "n_pending %d outside [n_clustered, n_total]", L->n_pending);
  return CKV_OK;
}

int check_ptrs(const char* names, int n, ...) {
  va_list ap;
  va_start(ap, n);
  for (int i = 0; i < n; ++i) {
    const void* p = va_arg(ap, const void*);
    if (!aligned16(p)) {
      va_end(ap);
      return fail(CKV_EINVAL, "pointer %d of (%s) is NULL or not 16-byte aligned", i, names);
    }
  }
  va_end(ap);
  return CKV_OK;
}

int check_ws(const ckv_layer* L, const void* ws, size_t ws_bytes, bool per_head = false) {
  if (!aligned16(ws)) return fail(CKV_EINVAL, "workspace is NULL or not 16-byte aligned");
  const Layout w = layout_of(L, per_head);
  if (ws_bytes < w.total)
    return fail(CKV_ENOSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  return CKV_OK;
}

int clustered_tokens(const ckv_layer* L) { return L->n_clustered - L->n_sink; }

// The kernels of one incremental clustering pass over the recent tokens
// [n_clustered, n_total): labels and running sums in place; the rebuilt index
// and scoring means go to offsets_out / cmean_out, the cluster-ordered copy to
// k_clu_alt / v_clu_alt.  Leaves *L unchanged.
int incremental_impl(const ckv_layer* L, void* ws, size_t ws_bytes, hipStream_t s, int32_t* offsets_out,
                     float* cmean_out) {
  int rc = check_ptrs("k_tok,v_tok,k_clu_alt,v_clu_alt,cdir,csum,msum,cmean,csize,offsets,assign,perm", 12,
                      L->k_tok, L->v_tok, L->k_clu_alt, L->v_clu_alt, L->cdir, L->csum, L->msum, cmean_out,
                      L->csize, offsets_out, L->assign, L->perm);
  if (rc) return rc;
  rc = check_ws(L, ws, ws_bytes);
  if (rc) return rc;
  const int units = L->batch * L->n_kv_heads;
  const int K = L->n_clusters;
  const int clu_stride = L->capacity - L->n_sink;
  const int m_old = L->n_clustered - L->n_sink;
  const int m_new = L->n_total - L->n_clustered;
  const int m = m_old + m_new;
  const Layout w = layout_of(L);
  double* invn = (double*)((char*)ws + w.off_invn);

  // the new keys' labels and inverse norms
  hipError_t e = ckv::launch_assign(L->k_tok, L->capacity, L->n_clustered, m_new, L->cdir, K, L->assign,
                                    clu_stride, m_old, units, s, invn);
  if (e != hipSuccess) return hip_status(e, "assign");
  e = ckv::launch_index(L->assign, clu_stride, m, K, L->n_sink, L->perm, offsets_out, units, s);
  if (e != hipSuccess) return hip_status(e, "index");
  e = ckv::launch_update(ckv::kUpdIncr, L->k_tok, L->v_tok, L->capacity, L->n_sink, L->perm, clu_stride,
                         offsets_out, K, invn, L->csum, L->msum, cmean_out, L->csize, L->cdir, L->k_clu_alt,
                         L->v_clu_alt, units, s);
  if (e != hipSuccess) return hip_status(e, "update");
  return CKV_OK;
}

}  // namespace

extern "C" {

const char* ckv_last_error(void) { return g_err; }

size_t ckv_abi_layer_bytes(void) { return sizeof(ckv_layer); }

size_t ckv_workspace_bytes(const ckv_layer* L, int32_t max_budget) {
  if (check_layer(L) != CKV_OK) return 0;
  if (max_budget < 0) {
    fail(CKV_EINVAL, "max_budget %d < 0", max_budget);
    return 0;
  }
  return layout_of(L).total;
}

int ckv_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!aligned16(ws)) return fail(CKV_EINVAL, "workspace is NULL or not 16-byte aligned");
  if (ws_bytes == 0) return fail(CKV_EINVAL, "ws_bytes is 0");
  return hip_status(ckv::launch_zero(ws, ws_bytes, (hipStream_t)stream), "workspace init");
}

}  // extern "C"

namespace {

// Checks of a prefill call (everything but the initial indices).
int prefill_check(ckv_layer* L, int32_t n, int32_t iters, void* ws, size_t ws_bytes) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (iters < 1) return fail(CKV_EINVAL, "iters %d < 1", iters);
  if (n > L->capacity) return fail(CKV_EINVAL, "n %d > capacity %d", n, L->capacity);
  if (L->n_pending != 0)
    return fail(CKV_EINVAL, "an asynchronous incremental call is pending (n_pending %d): commit it first",
                L->n_pending);
  const int m = n - L->n_sink;
  if (m < L->n_clusters) return fail(CKV_EINVAL, "need n_clusters %d <= m = n - n_sink = %d", L->n_clusters, m);
  rc = check_ptrs("k_tok,v_tok,k_clu,v_clu,cdir,csum,msum,cmean,csize,offsets,assign,perm", 12, L->k_tok, L->v_tok,
                  L->k_clu, L->v_clu, L->cdir, L->csum, L->msum, L->cmean, L->csize, L->offsets, L->assign, L->perm);
  if (rc) return rc;
  return check_ws(L, ws, ws_bytes);
}

// The prefill's kernels from the initial indices init_idx [units, K] on.
int prefill_run(ckv_layer* L, int32_t n, int32_t iters, const int32_t* init_idx, void* ws, hipStream_t s) {
  const int m = n - L->n_sink;
  const int units = L->batch * L->n_kv_heads;
  const int K = L->n_clusters;
  const int clu_stride = L->capacity - L->n_sink;
  const Layout w = layout_of(L);
  double* invn = (double*)((char*)ws + w.off_invn);

  hipError_t e = ckv::launch_init_dirs(L->k_tok, L->capacity, L->n_sink, m, init_idx, K, L->cdir, units, s);
  if (e != hipSuccess) return hip_status(e, "init");
  // Rounds between the first and the last move the sums by the keys that
  // changed cluster where the shape allows it; otherwise every round rebuilds
  // from the index.  Those rounds' labels alternate between two 16-bit
  // buffers in the workspace (the first round writes one of them beside
  // assign); the first and the last round write assign, which the index reads.
  const int stride16 = label16_stride(L);
  uint16_t* lab16 = (uint16_t*)((char*)ws + w.off_labs);
  const bool by_changes = ckv::delta_supported(K, m, units);
  for (int it = 0; it < iters; ++it) {
    const bool last = it == iters - 1;
    const bool middle = by_changes && !last && it > 0;
    uint16_t* cur16 = lab16 + (size_t)(it % 2) * units * stride16;
    uint16_t* prev16 = lab16 + (size_t)((it + 1) % 2) * units * stride16;
    // the first round's assignment also writes the keys' inverse norms
    e = ckv::launch_assign(L->k_tok, L->capacity, L->n_sink, m, L->cdir, K, middle ? nullptr : L->assign,
                           clu_stride, 0, units, s, it == 0 ? invn : nullptr,
                           (by_changes && !last) ? cur16 : nullptr, stride16);
    if (e != hipSuccess) return hip_status(e, "assign");
    if (middle) {
      e = ckv::launch_delta(cur16, prev16, stride16, clu_stride, m, K, L->k_tok, L->capacity, L->n_sink, invn,
                            L->csum, L->csize, L->cdir, units, s);
      if (e != hipSuccess) return hip_status(e, "delta update");
      continue;
    }
    // index, then the sums and directions from scratch (the first of rounds by
    // changes keeps them as fixed-point sums); the last round also writes the
    // means and the cluster-ordered rows
    e = ckv::launch_index(L->assign, clu_stride, m, K, L->n_sink, L->perm, L->offsets, units, s);
    if (e != hipSuccess) return hip_status(e, "index");
    const int mode = last ? ckv::kUpdFinal : (by_changes ? ckv::kUpdFixed : ckv::kUpdIter);
    e = ckv::launch_update(mode, L->k_tok, L->v_tok, L->capacity, L->n_sink, L->perm, clu_stride, L->offsets, K, invn,
                           L->csum, L->msum, L->cmean, L->csize, L->cdir, L->k_clu, L->v_clu, units, s, m);
    if (e != hipSuccess) return hip_status(e, "update");
  }
  L->n_total = n;
  L->n_clustered = n;
  return CKV_OK;
}

}  // namespace

extern "C" {

int ckv_init_indices(const ckv_layer* L, int32_t n, uint64_t seed, int32_t* init_idx, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (n > L->capacity) return fail(CKV_EINVAL, "n %d > capacity %d", n, L->capacity);
  const int m = n - L->n_sink;
  if (m < L->n_clusters) return fail(CKV_EINVAL, "need n_clusters %d <= m = n - n_sink = %d", L->n_clusters, m);
  rc = check_ptrs("init_idx", 1, init_idx);
  if (rc) return rc;
  const hipError_t e =
      ckv::launch_init_draw(seed, m, L->n_clusters, init_idx, L->batch * L->n_kv_heads, (hipStream_t)stream);
  return hip_status(e, "init draw");
}

int ckv_cluster_prefill(ckv_layer* L, int32_t n, int32_t iters, uint64_t seed, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc = prefill_check(L, n, iters, ws, ws_bytes);
  if (rc) return rc;
  // the drawn indices live in the auxiliary region, read once by the centre initialisation
  const Layout w = layout_of(L);
  int32_t* idx = (int32_t*)((char*)ws + w.off_aux);
  const hipStream_t s = (hipStream_t)stream;
  const hipError_t e = ckv::launch_init_draw(seed, n - L->n_sink, L->n_clusters, idx, L->batch * L->n_kv_heads, s);
  if (e != hipSuccess) return hip_status(e, "init draw");
  return prefill_run(L, n, iters, idx, ws, s);
}

int ckv_cluster_prefill_indices(ckv_layer* L, int32_t n, int32_t iters, const int32_t* init_idx, void* ws,
                                size_t ws_bytes, void* stream) {
  int rc = prefill_check(L, n, iters, ws, ws_bytes);
  if (rc) return rc;
  rc = check_ptrs("init_idx", 1, init_idx);
  if (rc) return rc;
  return prefill_run(L, n, iters, init_idx, ws, (hipStream_t)stream);
}

int ckv_append(ckv_layer* L, const uint16_t* k_new, const uint16_t* v_new, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  rc = check_ptrs("k_tok,v_tok,k_new,v_new", 4, L->k_tok, L->v_tok, k_new, v_new);
  if (rc) return rc;
  if (L->n_total >= L->capacity) return fail(CKV_ENOSPACE, "cache full (capacity %d)", L->capacity);
  const int units = L->batch * L->n_kv_heads;
  hipError_t e = ckv::launch_append(k_new, v_new, L->k_tok, L->v_tok, L->capacity, L->n_total, units,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "append");
  L->n_total += 1;
  return CKV_OK;
}

int ckv_cluster_incremental(ckv_layer* L, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (L->n_pending != 0)
    return fail(CKV_EINVAL, "an asynchronous incremental call is pending (n_pending %d): commit it first",
                L->n_pending);
  if (L->n_clustered < L->n_sink) return fail(CKV_EINVAL, "no cluster state (n_clustered < n_sink)");
  if (L->n_total == L->n_clustered) return CKV_OK;
  rc = incremental_impl(L, ws, ws_bytes, (hipStream_t)stream, L->offsets, L->cmean);
  if (rc) return rc;
  uint16_t* tk = L->k_clu;
  uint16_t* tv = L->v_clu;
  L->k_clu = L->k_clu_alt;
  L->v_clu = L->v_clu_alt;
  L->k_clu_alt = tk;
  L->v_clu_alt = tv;
  L->n_clustered = L->n_total;
  return CKV_OK;
}

int ckv_cluster_incremental_async(ckv_layer* L, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (L->n_pending != 0)
    return fail(CKV_EINVAL, "an asynchronous incremental call is already pending (n_pending %d)", L->n_pending);
  if (L->n_clustered < L->n_sink) return fail(CKV_EINVAL, "no cluster state (n_clustered < n_sink)");
  rc = check_ptrs("offsets_alt,cmean_alt", 2, L->offsets_alt, L->cmean_alt);
  if (rc) return rc;
  if (L->n_total == L->n_clustered) return CKV_OK;
  rc = incremental_impl(L, ws, ws_bytes, (hipStream_t)stream, L->offsets_alt, L->cmean_alt);
  if (rc) return rc;
  L->n_pending = L->n_total;
  return CKV_OK;
}

int ckv_cluster_commit(ckv_layer* L) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (L->n_pending == 0) return fail(CKV_EINVAL, "no asynchronous incremental call is pending");
  if (L->n_pending < L->n_clustered || L->n_pending > L->n_total)
    return fail(CKV_EINVAL, "n_pending %d outside [n_clustered, n_total]", L->n_pending);
  int32_t* to = L->offsets;
  L->offsets = L->offsets_alt;
  L->offsets_alt = to;
  float* tm = L->cmean;
  L->cmean = L->cmean_alt;
  L->cmean_alt = tm;
  uint16_t* tk = L->k_clu;
  uint16_t* tv = L->v_clu;
  L->k_clu = L->k_clu_alt;
  L->v_clu = L->v_clu_alt;
  L->k_clu_alt = tk;
  L->v_clu_alt = tv;
  L->n_clustered = L->n_pending;
  L->n_pending = 0;
  return CKV_OK;
}

int ckv_assign(const ckv_layer* L, int32_t n, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (n > L->capacity) return fail(CKV_EINVAL, "n %d > capacity %d", n, L->capacity);
  if (n <= L->n_sink) return fail(CKV_EINVAL, "n %d <= n_sink %d: no clustered token", n, L->n_sink);
  if (L->n_pending != 0)
    return fail(CKV_EINVAL, "an asynchronous incremental call is pending (n_pending %d): commit it first",
                L->n_pending);
  rc = check_ptrs("k_tok,cdir,assign", 3, L->k_tok, L->cdir, L->assign);
  if (rc) return rc;
  const int units = L->batch * L->n_kv_heads;
  const hipError_t e = ckv::launch_assign(L->k_tok, L->capacity, L->n_sink, n - L->n_sink, L->cdir, L->n_clusters,
                                          L->assign, L->capacity - L->n_sink, 0, units, (hipStream_t)stream);
  return hip_status(e, "assign");
}

int ckv_cluster_split(ckv_layer* L, double threshold, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (threshold != threshold) return fail(CKV_EINVAL, "threshold is NaN");
  if (L->n_pending != 0)
    return fail(CKV_EINVAL, "an asynchronous incremental call is pending (n_pending %d): commit it first",
                L->n_pending);
  if (L->n_clustered < L->n_sink) return fail(CKV_EINVAL, "no cluster state (n_clustered < n_sink)");
  rc = check_ptrs("k_tok,v_tok,k_clu,v_clu,cdir,csum,msum,cmean,csize,offsets,assign,perm", 12, L->k_tok,
                  L->v_tok, L->k_clu, L->v_clu, L->cdir, L->csum, L->msum, L->cmean, L->csize, L->offsets,
                  L->assign, L->perm);
  if (rc) return rc;
  rc = check_ws(L, ws, ws_bytes);
  if (rc) return rc;
  const int m = L->n_clustered - L->n_sink;
  if (m == 0) return CKV_OK;
  const hipStream_t s = (hipStream_t)stream;
  const int units = L->batch * L->n_kv_heads;
  const int K = L->n_clusters;
  const int clu_stride = L->capacity - L->n_sink;
  const Layout w = layout_of(L);

  // The pair plan, units x (2K + 1) int32, fills the auxiliary region, which
  // the rebuild below does not use.
  int32_t* plan = (int32_t*)((char*)ws + w.off_aux);
  hipError_t e = ckv::launch_split(L->k_clu, L->n_sink, L->perm, clu_stride, L->offsets, K, L->csum,
                                   L->csize, L->cdir, threshold, plan, L->assign, units, s);
  if (e != hipSuccess) return hip_status(e, "split");
  // one pass over the keys follows: the update takes each key's norm from the row itself
  e = ckv::launch_index(L->assign, clu_stride, m, K, L->n_sink, L->perm, L->offsets, units, s);
  if (e != hipSuccess) return hip_status(e, "index");
  e = ckv::launch_update(ckv::kUpdFinal, L->k_tok, L->v_tok, L->capacity, L->n_sink, L->perm, clu_stride,
                         L->offsets, K, nullptr, L->csum, L->msum, L->cmean, L->csize, L->cdir, L->k_clu, L->v_clu,
                         units, s);
  if (e != hipSuccess) return hip_status(e, "update");
  return CKV_OK;
}

}  // extern "C"

namespace {

int select_impl(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos, int32_t* sel_count,
                void* ws, size_t ws_bytes, void* stream, const uint16_t* k_new, const uint16_t* v_new,
                bool per_head = false) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (budget < 0) return fail(CKV_EINVAL, "budget %d < 0", budget);
  if (clustered_tokens(L) < L->n_clusters)
    return fail(CKV_EINVAL, "no cluster state: clustered tokens %d < n_clusters %d", clustered_tokens(L),
                L->n_clusters);
  rc = check_ptrs("q,cmean,offsets,k_clu,sel_count", 5, q, L->cmean, L->offsets, L->k_clu, sel_count);
  if (rc) return rc;
  if (budget > 0 && !aligned16(sel_pos)) return fail(CKV_EINVAL, "sel_pos is NULL or not 16-byte aligned");
  if (k_new != nullptr) {
    rc = check_ptrs("k_tok,v_tok,k_new,v_new", 4, L->k_tok, L->v_tok, k_new, v_new);
    if (rc) return rc;
    if (L->n_total >= L->capacity) return fail(CKV_ENOSPACE, "cache full (capacity %d)", L->capacity);
  }
  rc = check_ws(L, ws, ws_bytes, per_head);
  if (rc) return rc;
  const Layout w = layout_of(L, per_head);
  const int units = L->batch * L->n_kv_heads;
  const int sets = units * (per_head ? L->group : 1);
  hipError_t e = ckv::launch_select(q, L->group, L->cmean, L->offsets, L->n_clusters, L->k_clu,
                                    L->capacity - L->n_sink, budget, sel_pos, sel_count,
                                    (float*)((char*)ws + w.off_scores), (uint32_t*)((char*)ws + w.off_cut),
                                    (uint32_t*)ws + sets, k_new, v_new, L->k_tok, L->v_tok, L->capacity,
                                    L->n_total, units, per_head ? 1 : 0, (hipStream_t)stream);
  return hip_status(e, "select");
}

int decode_impl(const ckv_layer* L, const uint16_t* q, const int32_t* sel_pos, const int32_t* sel_count,
                int32_t budget, float* out, void* ws, size_t ws_bytes, void* stream, bool per_head) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (budget < 0) return fail(CKV_EINVAL, "budget %d < 0", budget);
  if (L->n_clustered < L->n_sink)
    return fail(CKV_EINVAL, "n_clustered %d < n_sink %d: cluster the prefix first", L->n_clustered, L->n_sink);
  rc = check_ptrs("q,k_tok,v_tok,sel_count,out", 5, q, L->k_tok, L->v_tok, sel_count, out);
  if (rc) return rc;
  const int m = clustered_tokens(L) > 0 ? clustered_tokens(L) : 0;
  const int cmax = budget < m ? budget : m;
  if (cmax > 0) {
    rc = check_ptrs("sel_pos,k_clu,v_clu", 3, sel_pos, L->k_clu, L->v_clu);
    if (rc) return rc;
  }
  rc = check_ws(L, ws, ws_bytes, per_head);
  if (rc) return rc;
  const int units = L->batch * L->n_kv_heads;
  const int sets = units * (per_head ? L->group : 1);
  const long long rmax = (long long)L->n_sink + cmax + (L->n_total - L->n_clustered);
  // Split-K: about kDecodeTargetWgs workgroups per launch (all resident at once
  // on 256 CUs), chunks of whole 16-row steps, at most kMaxChunks per unit.
#ifndef CKV_DEC_TARGET_WGS
#define CKV_DEC_TARGET_WGS 256
#endif
  const long long target = CKV_DEC_TARGET_WGS;
  long long chunk = (rmax * sets + target - 1) / target;
  const long long min_chunk = (rmax + ckv::kMaxChunks - 1) / ckv::kMaxChunks;
  if (chunk < min_chunk) chunk = min_chunk;
  if (chunk < 64) chunk = 64;
  chunk = (chunk + 15) / 16 * 16;
  long long n_chunks = (rmax + chunk - 1) / chunk;
  if (n_chunks < 1) n_chunks = 1;
  const Layout w = layout_of(L, per_head);
  hipError_t e = ckv::launch_sparse_decode(
      q, L->group, L->k_tok, L->v_tok, L->capacity, L->k_clu, L->v_clu, L->capacity - L->n_sink, sel_pos,
      sel_count, budget, m, L->n_sink, L->n_clustered, L->n_total, (int)chunk, (int)n_chunks,
      (float*)((char*)ws + w.off_partials), (uint32_t*)ws, out, units, per_head ? 1 : 0, (hipStream_t)stream);
  return hip_status(e, "sparse_decode");
}

// Checks shared by the fused recall + decode calls (everything but the scratch).
int select_decode_check(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                        int32_t* sel_count, float* out, const uint16_t* k_new, const uint16_t* v_new) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (budget < 0) return fail(CKV_EINVAL, "budget %d < 0", budget);
  if (clustered_tokens(L) < L->n_clusters)
    return fail(CKV_EINVAL, "no cluster state: clustered tokens %d < n_clusters %d", clustered_tokens(L),
                L->n_clusters);
  rc = check_ptrs("q,cmean,offsets,k_tok,v_tok,k_clu,v_clu,sel_count,out", 9, q, L->cmean, L->offsets, L->k_tok,
                  L->v_tok, L->k_clu, L->v_clu, sel_count, out);
  if (rc) return rc;
  if (budget > 0 && !aligned16(sel_pos)) return fail(CKV_EINVAL, "sel_pos is NULL or not 16-byte aligned");
  if (k_new != nullptr) {
    rc = check_ptrs("k_new,v_new", 2, k_new, v_new);
    if (rc) return rc;
    if (L->n_total >= L->capacity) return fail(CKV_ENOSPACE, "cache full (capacity %d)", L->capacity);
  }
  return CKV_OK;
}

// The fused launch over caller-provided scratch: split-K partials, arrival
// counters (zero on entry, left zero) and the cut-cluster score area.
int select_decode_launch(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                         int32_t* sel_count, float* out, void* stream, const uint16_t* k_new, const uint16_t* v_new,
                         bool per_head, const ckv_layer* next, float* partials, uint32_t* counters,
                         uint32_t* cut_scores) {
  const int units = L->batch * L->n_kv_heads;
  const int n_total = L->n_total + (k_new != nullptr ? 1 : 0);
  // the prefetch hint is used only for a layer laid out like this one
  const float* pf_cmean = nullptr;
  const int32_t* pf_offsets = nullptr;
  if (next != nullptr && next->batch == L->batch && next->n_kv_heads == L->n_kv_heads &&
      next->n_clusters == L->n_clusters && aligned16(next->cmean) && aligned16(next->offsets)) {
    pf_cmean = next->cmean;
    pf_offsets = next->offsets;
  }
  hipError_t e = ckv::launch_recall_decode(
      q, L->group, L->cmean, L->offsets, L->n_clusters, L->k_tok, L->v_tok, L->capacity, L->k_clu, L->v_clu,
      L->capacity - L->n_sink, budget, L->n_sink, L->n_clustered, n_total, sel_pos, sel_count, partials, counters,
      cut_scores, out, k_new, v_new, pf_cmean, pf_offsets, units, per_head ? 1 : 0, (hipStream_t)stream);
  return hip_status(e, "select_decode");
}

int select_decode_impl(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                       int32_t* sel_count, float* out, void* ws, size_t ws_bytes, void* stream,
                       const uint16_t* k_new, const uint16_t* v_new, bool per_head, const ckv_layer* next) {
  int rc = select_decode_check(L, q, budget, sel_pos, sel_count, out, k_new, v_new);
  if (rc) return rc;
  rc = check_ws(L, ws, ws_bytes, per_head);
  if (rc) return rc;
  const Layout w = layout_of(L, per_head);
  return select_decode_launch(L, q, budget, sel_pos, sel_count, out, stream, k_new, v_new, per_head, next,
                              (float*)((char*)ws + w.off_partials), (uint32_t*)ws,
                              (uint32_t*)((char*)ws + w.off_rd_cut));
}

}  // namespace

extern "C" {

int ckv_select_decode(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos, int32_t* sel_count,
                      float* out, const ckv_layer* next, void* ws, size_t ws_bytes, void* stream) {
  return select_decode_impl(L, q, budget, sel_pos, sel_count, out, ws, ws_bytes, stream, nullptr, nullptr, false,
                            next);
}

int ckv_append_select_decode(ckv_layer* L, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                             int32_t budget, int32_t* sel_pos, int32_t* sel_count, float* out, const ckv_layer* next,
                             void* ws, size_t ws_bytes, void* stream) {
  if (k_new == nullptr || v_new == nullptr) return fail(CKV_EINVAL, "k_new / v_new is NULL");
  const int rc =
      select_decode_impl(L, q, budget, sel_pos, sel_count, out, ws, ws_bytes, stream, k_new, v_new, false, next);
  if (rc) return rc;
  L->n_total += 1;
  return CKV_OK;
}

int ckv_select_decode_per_head(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                               int32_t* sel_count, float* out, const ckv_layer* next, void* ws, size_t ws_bytes,
                               void* stream) {
  return select_decode_impl(L, q, budget, sel_pos, sel_count, out, ws, ws_bytes, stream, nullptr, nullptr, true,
                            next);
}

int ckv_select(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos, int32_t* sel_count,
               void* ws, size_t ws_bytes, void* stream) {
  return select_impl(L, q, budget, sel_pos, sel_count, ws, ws_bytes, stream, nullptr, nullptr);
}

int ckv_append_select(ckv_layer* L, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                      int32_t budget, int32_t* sel_pos, int32_t* sel_count, void* ws, size_t ws_bytes,
                      void* stream) {
  if (k_new == nullptr || v_new == nullptr) return fail(CKV_EINVAL, "k_new / v_new is NULL");
  const int rc = select_impl(L, q, budget, sel_pos, sel_count, ws, ws_bytes, stream, k_new, v_new);
  if (rc) return rc;
  L->n_total += 1;
  return CKV_OK;
}


int ckv_sparse_decode(const ckv_layer* L, const uint16_t* q, const int32_t* sel_pos, const int32_t* sel_count,
                      int32_t budget, float* out, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(L, q, sel_pos, sel_count, budget, out, ws, ws_bytes, stream, false);
}

size_t ckv_workspace_bytes_per_head(const ckv_layer* L, int32_t max_budget) {
  if (check_layer(L)) return 0;
  if (max_budget < 0) {
    fail(CKV_EINVAL, "max_budget %d < 0", max_budget);
    return 0;
  }
  return layout_of(L, true).total;
}

int ckv_select_per_head(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                        int32_t* sel_count, void* ws, size_t ws_bytes, void* stream) {
  return select_impl(L, q, budget, sel_pos, sel_count, ws, ws_bytes, stream, nullptr, nullptr, true);
}

int ckv_sparse_decode_per_head(const ckv_layer* L, const uint16_t* q, const int32_t* sel_pos,
                               const int32_t* sel_count, int32_t budget, float* out, void* ws, size_t ws_bytes,
                               void* stream) {
  return decode_impl(L, q, sel_pos, sel_count, budget, out, ws, ws_bytes, stream, true);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The allocation-free fused call: its scratch lives in a file-scope device
// array instead of a caller workspace.  Each device holds its own copy of the
// array until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
constexpr size_t kNoAllocCounterBytes = (size_t)64 << 10;  // arrival counters: up to 16384 sets
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
bool g_scratch_cleared[kMaxDevices];        // its counters zero-filled on that device

// Bytes of scratch one ckv_select_decode_noalloc call needs: the counters,
// then the split-K partials, then the cut-cluster score area.
size_t noalloc_bytes(const ckv_layer* L, int32_t budget) {
  const size_t units = (size_t)L->batch * L->n_kv_heads;
  const int m = clustered_tokens(L);
  const int beff = budget < m ? budget : m;
  const int rows = L->n_sink + beff + (L->n_total - L->n_clustered);
  const int W = ckv::recall_decode_chunks((int)units, rows);
  const size_t partials = align256(units * W * group_tier(L->group) * ckv::kPartialStride * sizeof(float));
  const size_t cut = align256(units * (size_t)(L->capacity - L->n_sink) * sizeof(uint32_t));
  return kNoAllocCounterBytes + partials + cut;
}

// The scratch of the current device; the first call on a device looks up its
// address and zero-fills the counters on `s` (with a kernel, so a caller may
// capture it in a graph).
int noalloc_scratch(hipStream_t s, unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CKV_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(CKV_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = (unsigned char*)p;
  }
  if (!g_scratch_cleared[dev]) {
    e = ckv::launch_zero(g_scratch_ptr[dev], kNoAllocCounterBytes, s);
    if (e != hipSuccess) return hip_status(e, "zero-fill of the no-alloc counters");
    g_scratch_cleared[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return CKV_OK;
}

}  // namespace

extern "C" {

size_t ckv_select_decode_noalloc_limit(void) { return kNoAllocScratchBytes; }

int ckv_select_decode_noalloc(const ckv_layer* L, const uint16_t* q, int32_t budget, int32_t* sel_pos,
                              int32_t* sel_count, float* out, const ckv_layer* next, void* stream) {
  int rc = select_decode_check(L, q, budget, sel_pos, sel_count, out, nullptr, nullptr);
  if (rc) return rc;
  const size_t units = (size_t)L->batch * L->n_kv_heads;
  if (units * sizeof(uint32_t) > kNoAllocCounterBytes)
    return fail(CKV_ENOSPACE, "no-alloc call: %zu units exceed the %zu counters", units,
                kNoAllocCounterBytes / sizeof(uint32_t));
  const size_t need = noalloc_bytes(L, budget);
  if (need > kNoAllocScratchBytes)
    return fail(CKV_ENOSPACE, "no-alloc call needs %zu bytes of scratch > the %zu-byte limit", need,
                kNoAllocScratchBytes);
  const int m = clustered_tokens(L);
  const int beff = budget < m ? budget : m;
  const int W = ckv::recall_decode_chunks((int)units, L->n_sink + beff + (L->n_total - L->n_clustered));
  const size_t partial_bytes = align256(units * W * group_tier(L->group) * ckv::kPartialStride * sizeof(float));
  unsigned char* base = nullptr;
  rc = noalloc_scratch((hipStream_t)stream, &base);
  if (rc) return rc;
  return select_decode_launch(L, q, budget, sel_pos, sel_count, out, stream, nullptr, nullptr, false, next,
                              (float*)(base + kNoAllocCounterBytes), (uint32_t*)base,
                              (uint32_t*)(base + kNoAllocCounterBytes + partial_bytes));
}

}  // extern "C"
