"""Oracle: a plain, slow, float64 CPU implementation of the ClusterKV hot path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product (the HIP library ``libckv.so`` and its Python binding) never imports,
links or runs it, and shares no code, table or helper with it.

Pages followed (cited by title and section; no other source):

* "ClusterKV article" -- the intelliparadigm.com article
  "大模型KV Cache压缩技术：ClusterKV的语义空间优化" (a write-up of the DAC'25
  paper "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
  Recallable Compression").  Sections used: §3.1 (attention and the centroid
  approximation), §3.2 (prefill clustering, incremental clustering), §3.3
  (cluster selection procedure), §4.1 (cluster-contiguous KV layout).
* "ClusterKV abstract" -- the arxivdaily.com listing of arXiv 2412.03213
  (recall at semantic-cluster granularity; clustering, selection, indexing and
  caching as the four stages).

Arithmetic: every input is a bfloat16 value widened exactly to float64; all
oracle arithmetic is float64.  The only rounding the method itself performs is
the bfloat16 rounding of the unit-direction centroids (``bf16.round_rne``),
which the oracle applies directly from float64.

Where the pages leave a step open the oracle takes one reading; the readings
are listed in each function's docstring.

Pins (what each function is checked against, in ``tests/test_oracle_*.py``):
``bf16`` -- exact-rational rounding on sampled values and agreement with the
float32 route on float32-representable values; ``kmeans.assign`` --
brute-force ``fsum`` argmax, scale invariance, K = 1, planted ties;
``kmeans.lloyd`` -- objective monotonicity in exact mode, the rounding bound in
bf16 mode, a fixed point, brute-force optimum on tiny inputs, a hand-worked
golden example; ``kmeans.build_index`` -- bijection / scan / stability;
``kmeans.scoring_centroids`` -- Jensen's inequality, the tight-cluster limit
and the Gaussian closed form of the centroid approximation (§3.1);
``init.init_indices`` -- published SplitMix64 outputs, a hand-worked Floyd
draw, distinctness, range, determinism and uniformity over subsets;
``select.select_unit`` -- a hand-worked golden example, an independent
total-order formulation, exact count, prefix property, budget >= m;
``attention.attend`` -- torch's float64 SDPA, |S| = 1, q = 0, order and shift
invariance, a hand-worked golden example; ``kmeans.incremental`` --
brute-force assignment and from-scratch recomputation of the running sums;
``kmeans.drift`` -- the brute-force mean distance over the members, identical
and antipodal members; ``kmeans.split`` -- two planted groups separated
exactly, no change above the largest drift or without an empty slot, the most
drifted cluster served first, drift ties, seed ties, label and size
invariants; reserved slots -- Lloyd with reserves equals Lloyd without them
when no key is an outlier, and an outlier lands in the reserve.
"""

from . import bf16, kmeans, select, attention, pipeline, init  # noqa: F401
