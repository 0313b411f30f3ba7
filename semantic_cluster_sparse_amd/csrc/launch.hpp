// Internal launch interface between the C-ABI layer (api.hip) and the kernel
// translation units.  Every launcher only enqueues on `s` and returns the
// launch status; argument validation happens in api.hip before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckv {

constexpr int kMaxClusters = 1024;  // K limit of the LDS-resident per-cluster arrays
constexpr int kMaxGroup = 16;
constexpr int kMaxChunks = 64;      // split-K chunks per unit in sparse decode
constexpr int kPartialStride = 130; // floats per (chunk, head) partial: o[128], m, l

enum UpdateMode { kUpdIter = 0, kUpdFinal = 1, kUpdIncr = 2, kUpdFixed = 3 };

// init_idx[u, 0:K] = Floyd's sample of K distinct indices in [0, m) driven
// by SplitMix64 from state seed + u (K <= kMaxClusters, K <= m).
hipError_t launch_init_draw(uint64_t seed, int m, int K, int32_t* init_idx, int units, hipStream_t s);

// c_j = bf16(x_idx / |x_idx|) for idx = init_idx[u, j] (zero if idx outside [0, m)).
hipError_t launch_init_dirs(const uint16_t* k_tok, int capacity, int n_sink, int m,
                            const int32_t* init_idx, int K, uint16_t* cdir, int units,
                            hipStream_t s);

// assign[u, first + i] = argmax_j k_tok[u, row0 + i] . cdir[u, j] for i < count.
// With invn non-null also invn[u, first + i] = 1/|k_tok[u, row0 + i]| (f64),
// the same values launch_inv_norm writes.
// assign16 (uint16, row stride stride16; K <= 512 only) takes a copy of the
// labels, and assign may be null when only that copy is wanted.
hipError_t launch_assign(const uint16_t* k_tok, int capacity, int row0, int count,
                         const uint16_t* cdir, int K, int32_t* assign, int clu_stride,
                         int first, int units, hipStream_t s, double* invn = nullptr,
                         uint16_t* assign16 = nullptr, int stride16 = 0);

// 1/|x| (f64) of clustered tokens [first, first + count) into invn[u, first + i].
hipError_t launch_inv_norm(const uint16_t* k_tok, int capacity, int n_sink, int first, int count,
                           double* invn, int clu_stride, int units, hipStream_t s);

// Stable counting sort by label in one launch: perm[u, pos] = n_sink + i in
// cluster order (token order inside a cluster), offsets[u, 0..K].
hipError_t launch_index(const int32_t* assign, int clu_stride, int count, int K, int n_sink, int32_t* perm,
                        int32_t* offsets, int units, hipStream_t s);

// A Lloyd round between the first and the last from the keys that changed
// cluster between prev_lab and cur_lab (uint16 labels, row stride stride16,
// even and >= count; columns 0:count).  While the rounds run, csum holds the
// unit-key sums as int64 fixed point (the first round's kUpdFixed update
// writes them, the last round's update writes them in f64 again); csize and
// cdir are kept current.  invn[u, i] (row stride clu_stride) = 1/|x_i| of
// every clustered token.  delta_supported says whether a shape takes this
// form (else every round rebuilds from the index).
bool delta_supported(int K, int count, int units);
hipError_t launch_delta(const uint16_t* cur_lab, const uint16_t* prev_lab, int stride16, int clu_stride, int count,
                        int K, const uint16_t* k_tok, int capacity, int n_sink, const double* invn, double* csum,
                        int32_t* csize, uint16_t* cdir, int units, hipStream_t s);

// Per-cluster segmented reduction over the members listed by perm/offsets.
// kUpdFixed writes csum as the int64 fixed-point sums of launch_delta (count =
// the clustered keys per unit, which fixes the scale).
hipError_t launch_update(int mode, const uint16_t* k_tok, const uint16_t* v_tok, int capacity,
                         int n_sink, const int32_t* perm, int clu_stride, const int32_t* offsets,
                         int K, const double* invn, double* csum, double* msum, float* cmean,
                         int32_t* csize, uint16_t* cdir, uint16_t* k_dst, uint16_t* v_dst,
                         int units, hipStream_t s, int count = 0);

// Drift split: the pairs go to plan [units, 2K + 1] int32 (workspace), then
// the labels of the split clusters' members are rewritten.
hipError_t launch_split(const uint16_t* k_clu, int n_sink, const int32_t* perm, int clu_stride,
                        const int32_t* offsets, int K, const double* csum, const int32_t* csize,
                        const uint16_t* cdir, double threshold, int32_t* plan, int32_t* assign, int units,
                        hipStream_t s);

// Recall: cluster scores (several workgroups per unit), then the last of them
// finds the cut, the partial top-k and writes the positions.  counters[units]
// must be zero on entry and are zero again on exit.  With k_new non-null the
// same launch also writes k_new / v_new into row `row` of k_tok / v_tok.
hipError_t launch_select(const uint16_t* q, int group, const float* cmean,
                         const int32_t* offsets, int K, const uint16_t* k_clu, int clu_stride,
                         int budget, int32_t* sel_pos, int32_t* sel_count, float* scores_ws,
                         uint32_t* cut_ws, uint32_t* counters, const uint16_t* k_new,
                         const uint16_t* v_new, uint16_t* k_tok, uint16_t* v_tok, int capacity, int row,
                         int units, int per_head, hipStream_t s);

// Split-K sparse decode streaming rows through per-wave LDS rings; the last
// chunk of each unit merges the chunk partials.  counters[units] must be zero
// on entry and are zero again on exit.
hipError_t launch_sparse_decode(const uint16_t* q, int group, const uint16_t* k_tok,
                                const uint16_t* v_tok, int capacity, const uint16_t* k_clu,
                                const uint16_t* v_clu, int clu_stride, const int32_t* sel_pos,
                                const int32_t* sel_count, int budget, int m, int n_sink,
                                int n_clustered, int n_total, int chunk_rows, int n_chunks,
                                float* partials, uint32_t* counters, float* out, int units,
                                int per_head, hipStream_t s);

// Chunks (workgroups) per attended set of a fused recall + decode launch over
// `sets` sets of `rows` attended rows each; its split-K partials take
// sets * chunks * group_tier * kPartialStride floats.
int recall_decode_chunks(int sets, int rows);

// Recall and sparse decode in one launch: every workgroup of a set recalls
// the set itself, then streams its chunk of the attended rows (sinks, recent
// rows, whole clusters, the cut's kept tokens) and the last chunk merges.
// Writes sel_pos / sel_count as launch_select does and out as
// launch_sparse_decode does.  counters[sets] must be zero on entry and are
// zero again on exit; cut_ws [sets, clu_stride] u32 is scratch for cut
// clusters above 4096 tokens.  With k_new non-null the launch also appends
// k_new / v_new as row n_total - 1 (n_total counts it) and attends to it.
// pf_cmean / pf_offsets (or null): centroids [units, K, 128] and offsets
// [units, K + 1] of the next call's layer, read into the caches at the end.
hipError_t launch_recall_decode(const uint16_t* q, int group, const float* cmean, const int32_t* offsets, int K,
                                uint16_t* k_tok, uint16_t* v_tok, int capacity, const uint16_t* k_clu,
                                const uint16_t* v_clu, int clu_stride, int budget, int n_sink, int n_clustered,
                                int n_total, int32_t* sel_pos, int32_t* sel_count, float* partials,
                                uint32_t* counters, uint32_t* cut_ws, float* out, const uint16_t* k_new,
                                const uint16_t* v_new, const float* pf_cmean, const int32_t* pf_offsets, int units,
                                int per_head, hipStream_t s);

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_tok,
                         uint16_t* v_tok, int capacity, int row, int units, hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace ckv
