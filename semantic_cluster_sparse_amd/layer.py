"""One layer's device buffers, allocated with PyTorch, and the calls on them.

``Layer`` owns the tensors a ``ckv_layer`` points at (token-order K/V, the
cluster-ordered copies, the centroid state and the index) plus a workspace,
and forwards to the C ABI through ``ckv``.  PyTorch only allocates memory and
supplies the current HIP stream; every step of the method runs in libckv.so.
"""

from __future__ import annotations

import torch

from . import ckv

HEAD_DIM = 128


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _struct(layer):
    return layer.struct if layer is not None else None


class Layer:
    def __init__(self, batch: int, n_kv_heads: int, group: int, n_clusters: int, capacity: int,
                 n_sink: int = 16, max_budget: int = 2048, incremental: bool = True, per_head: bool = False,
                 device: str | torch.device = "cuda"):
        self.device = torch.device(device)
        self.units = batch * n_kv_heads
        self.group = group
        self.n_sink = n_sink
        self.n_clusters = n_clusters
        self.capacity = capacity
        u, K, d = self.units, n_clusters, HEAD_DIM
        clu = capacity - n_sink
        bf = dict(dtype=torch.bfloat16, device=self.device)
        self.k_tok = torch.zeros((u, capacity, d), **bf)
        self.v_tok = torch.zeros((u, capacity, d), **bf)
        self.k_clu = torch.zeros((u, clu, d), **bf)
        self.v_clu = torch.zeros((u, clu, d), **bf)
        self.k_clu_alt = torch.zeros((u, clu, d), **bf) if incremental else None
        self.v_clu_alt = torch.zeros((u, clu, d), **bf) if incremental else None
        self.cdir = torch.zeros((u, K, d), **bf)
        self.csum = torch.zeros((u, K, d), dtype=torch.float64, device=self.device)
        self.msum = torch.zeros((u, K, d), dtype=torch.float64, device=self.device)
        self.cmean = torch.zeros((u, K, d), dtype=torch.float32, device=self.device)
        i32 = dict(dtype=torch.int32, device=self.device)
        self.csize = torch.zeros((u, K), **i32)
        self.offsets = torch.zeros((u, K + 1), **i32)
        self.assign = torch.zeros((u, clu), **i32)
        self.perm = torch.zeros((u, clu), **i32)
        # second index / means and a second workspace for clustering beside decoding
        self.offsets_alt = torch.zeros((u, K + 1), **i32) if incremental else None
        self.cmean_alt = torch.zeros((u, K, d), dtype=torch.float32, device=self.device) if incremental else None
        self.struct = ckv.CkvLayerStruct(
            batch=batch, n_kv_heads=n_kv_heads, group=group, head_dim=HEAD_DIM, n_sink=n_sink,
            n_clusters=n_clusters, capacity=capacity, n_total=0, n_clustered=0, n_pending=0)
        self._bind()
        # a per-query-head workspace also serves every other call
        self.ws_bytes = (ckv.ckv_workspace_bytes_per_head if per_head else ckv.ckv_workspace_bytes)(
            self.struct, max_budget)
        self.ws = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=self.device)
        ckv.ckv_workspace_init(self.ws.data_ptr(), self.ws_bytes, _stream())
        self.ws_bg = None
        if incremental:
            self.ws_bg = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=self.device)
            ckv.ckv_workspace_init(self.ws_bg.data_ptr(), self.ws_bytes, _stream())

    def _bind(self) -> None:
        s = self.struct
        for name in ("k_tok", "v_tok", "k_clu", "v_clu", "k_clu_alt", "v_clu_alt", "cdir", "csum",
                     "msum", "cmean", "csize", "offsets", "assign", "perm", "offsets_alt", "cmean_alt"):
            t = getattr(self, name)
            setattr(s, name, t.data_ptr() if t is not None else None)

    @property
    def n_total(self) -> int:
        return self.struct.n_total

    @property
    def n_clustered(self) -> int:
        return self.struct.n_clustered

    def set_counters(self, n_total: int, n_clustered: int) -> None:
        self.struct.n_total = n_total
        self.struct.n_clustered = n_clustered

    # ----------------------------------------------------------------- calls
    def prefill(self, n: int, iters: int, init) -> None:
        """Prefill clustering of tokens [n_sink, n): `init` is a seed (int; the
        library draws the initial indices, ckv_cluster_prefill) or the initial
        indices themselves (int32 [units, K] tensor, ckv_cluster_prefill_indices)."""
        if isinstance(init, int):
            ckv.ckv_cluster_prefill(self.struct, n, iters, init, self.ws.data_ptr(), self.ws_bytes, _stream())
            return
        assert init.dtype == torch.int32 and init.is_contiguous()
        assert tuple(init.shape) == (self.units, self.n_clusters)
        ckv.ckv_cluster_prefill_indices(self.struct, n, iters, init.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                                        _stream())

    def init_indices(self, n: int, seed: int) -> torch.Tensor:
        """The initial indices the seeded prefill of tokens [n_sink, n) draws (ckv_init_indices)."""
        out = torch.empty((self.units, self.n_clusters), dtype=torch.int32, device=self.device)
        ckv.ckv_init_indices(self.struct, n, seed, out.data_ptr(), _stream())
        return out

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        assert k_new.shape == (self.units, HEAD_DIM) and v_new.shape == (self.units, HEAD_DIM)
        assert k_new.is_contiguous() and v_new.is_contiguous()
        ckv.ckv_append(self.struct, k_new.data_ptr(), v_new.data_ptr(), _stream())

    def incremental(self) -> None:
        ckv.ckv_cluster_incremental(self.struct, self.ws.data_ptr(), self.ws_bytes, _stream())
        self._sync_swapped()

    def incremental_async(self) -> None:
        """Cluster the recent tokens into the second buffers, on the current stream,
        with the second workspace; recall and decode may go on meanwhile on another
        stream.  commit() makes the result current."""
        ckv.ckv_cluster_incremental_async(self.struct, self.ws_bg.data_ptr(), self.ws_bytes, _stream())

    def commit(self) -> None:
        ckv.ckv_cluster_commit(self.struct)
        self._sync_swapped()

    def _sync_swapped(self) -> None:
        # the library exchanged buffers inside the struct: follow it
        pairs = (("k_clu", "k_clu_alt"), ("v_clu", "v_clu_alt"), ("offsets", "offsets_alt"), ("cmean", "cmean_alt"))
        for cur, alt in pairs:
            t_cur, t_alt = getattr(self, cur), getattr(self, alt)
            if t_alt is not None and getattr(self.struct, cur) == t_alt.data_ptr():
                setattr(self, cur, t_alt)
                setattr(self, alt, t_cur)

    def assign_only(self, n: int) -> None:
        """The assignment step alone over tokens [n_sink, n): labels only."""
        ckv.ckv_assign(self.struct, n, _stream())

    def split(self, threshold: float) -> None:
        """Split drifted clusters into empty slots, then rebuild the index and rows in place."""
        ckv.ckv_cluster_split(self.struct, threshold, self.ws.data_ptr(), self.ws_bytes, _stream())

    @property
    def n_pending(self) -> int:
        return self.struct.n_pending

    def select(self, q: torch.Tensor, budget: int, sel_pos: torch.Tensor,
               sel_count: torch.Tensor) -> None:
        assert q.is_contiguous() and q.numel() == self.units * self.group * HEAD_DIM
        assert sel_pos.numel() >= self.units * budget and sel_count.numel() >= self.units
        ckv.ckv_select(self.struct, q.data_ptr(), budget, sel_pos.data_ptr(), sel_count.data_ptr(),
                       self.ws.data_ptr(), self.ws_bytes, _stream())

    def append_select(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, budget: int,
                      sel_pos: torch.Tensor, sel_count: torch.Tensor) -> None:
        assert k_new.shape == (self.units, HEAD_DIM) and v_new.shape == (self.units, HEAD_DIM)
        assert k_new.is_contiguous() and v_new.is_contiguous()
        assert q.is_contiguous() and q.numel() == self.units * self.group * HEAD_DIM
        assert sel_pos.numel() >= self.units * budget and sel_count.numel() >= self.units
        ckv.ckv_append_select(self.struct, k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), budget,
                              sel_pos.data_ptr(), sel_count.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                              _stream())

    def sparse_decode(self, q: torch.Tensor, sel_pos: torch.Tensor, sel_count: torch.Tensor,
                      budget: int, out: torch.Tensor) -> None:
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        assert out.numel() == self.units * self.group * HEAD_DIM
        ckv.ckv_sparse_decode(self.struct, q.data_ptr(), sel_pos.data_ptr(), sel_count.data_ptr(),
                              budget, out.data_ptr(), self.ws.data_ptr(), self.ws_bytes, _stream())

    def select_per_head(self, q: torch.Tensor, budget: int, sel_pos: torch.Tensor,
                        sel_count: torch.Tensor) -> None:
        assert q.is_contiguous() and q.numel() == self.units * self.group * HEAD_DIM
        assert sel_pos.numel() >= self.units * self.group * budget
        assert sel_count.numel() >= self.units * self.group
        ckv.ckv_select_per_head(self.struct, q.data_ptr(), budget, sel_pos.data_ptr(), sel_count.data_ptr(),
                                self.ws.data_ptr(), self.ws_bytes, _stream())

    def sparse_decode_per_head(self, q: torch.Tensor, sel_pos: torch.Tensor, sel_count: torch.Tensor,
                               budget: int, out: torch.Tensor) -> None:
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        assert out.numel() == self.units * self.group * HEAD_DIM
        ckv.ckv_sparse_decode_per_head(self.struct, q.data_ptr(), sel_pos.data_ptr(), sel_count.data_ptr(),
                                       budget, out.data_ptr(), self.ws.data_ptr(), self.ws_bytes, _stream())

    def select_decode(self, q: torch.Tensor, budget: int, sel_pos: torch.Tensor, sel_count: torch.Tensor,
                      out: torch.Tensor, next_layer: "Layer | None" = None) -> None:
        """Recall and decode in one launch (ckv_select_decode); next_layer is the
        prefetch hint (the layer whose call follows on the stream)."""
        assert q.is_contiguous() and q.numel() == self.units * self.group * HEAD_DIM
        assert sel_pos.numel() >= self.units * budget and sel_count.numel() >= self.units
        assert out.is_contiguous() and out.dtype == torch.float32 and out.numel() == self.units * self.group * HEAD_DIM
        ckv.ckv_select_decode(self.struct, q.data_ptr(), budget, sel_pos.data_ptr(), sel_count.data_ptr(),
                              out.data_ptr(), _struct(next_layer), self.ws.data_ptr(), self.ws_bytes, _stream())

    def append_select_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, budget: int,
                             sel_pos: torch.Tensor, sel_count: torch.Tensor, out: torch.Tensor,
                             next_layer: "Layer | None" = None) -> None:
        """Append the decoded token, recall and decode in one launch (ckv_append_select_decode)."""
        assert k_new.shape == (self.units, HEAD_DIM) and v_new.shape == (self.units, HEAD_DIM)
        assert k_new.is_contiguous() and v_new.is_contiguous()
        assert q.is_contiguous() and q.numel() == self.units * self.group * HEAD_DIM
        assert sel_pos.numel() >= self.units * budget and sel_count.numel() >= self.units
        assert out.is_contiguous() and out.dtype == torch.float32 and out.numel() == self.units * self.group * HEAD_DIM
        ckv.ckv_append_select_decode(self.struct, k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), budget,
                                     sel_pos.data_ptr(), sel_count.data_ptr(), out.data_ptr(), _struct(next_layer),
                                     self.ws.data_ptr(), self.ws_bytes, _stream())

    def select_decode_per_head(self, q: torch.Tensor, budget: int, sel_pos: torch.Tensor, sel_count: torch.Tensor,
                               out: torch.Tensor, next_layer: "Layer | None" = None) -> None:
        """Per-query-head recall and decode in one launch (ckv_select_decode_per_head)."""
        assert q.is_contiguous() and q.numel() == self.units * self.group * HEAD_DIM
        assert sel_pos.numel() >= self.units * self.group * budget
        assert sel_count.numel() >= self.units * self.group
        assert out.is_contiguous() and out.dtype == torch.float32 and out.numel() == self.units * self.group * HEAD_DIM
        ckv.ckv_select_decode_per_head(self.struct, q.data_ptr(), budget, sel_pos.data_ptr(), sel_count.data_ptr(),
                                       out.data_ptr(), _struct(next_layer), self.ws.data_ptr(), self.ws_bytes,
                                       _stream())

    def select_decode_noalloc(self, q: torch.Tensor, budget: int, sel_pos: torch.Tensor, sel_count: torch.Tensor,
                              out: torch.Tensor, next_layer: "Layer | None" = None) -> None:
        """ckv_select_decode without the workspace (the library's per-device scratch array)."""
        assert q.is_contiguous() and q.numel() == self.units * self.group * HEAD_DIM
        assert sel_pos.numel() >= self.units * budget and sel_count.numel() >= self.units
        assert out.is_contiguous() and out.dtype == torch.float32 and out.numel() == self.units * self.group * HEAD_DIM
        ckv.ckv_select_decode_noalloc(self.struct, q.data_ptr(), budget, sel_pos.data_ptr(), sel_count.data_ptr(),
                                      out.data_ptr(), _struct(next_layer), _stream())
