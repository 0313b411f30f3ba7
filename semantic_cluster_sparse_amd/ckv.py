"""ctypes binding of libckv.so: argument marshalling only.

Every function has the name of the C entry point it calls (``include/ckv.h``)
and raises ``CkvError`` when that call returns a nonzero code.  Device
pointers are plain integers (``tensor.data_ptr()``); ``stream`` is a HIP
stream handle as an integer (``torch.cuda.current_stream().cuda_stream``) or
0 for the default stream.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_int, c_int32, c_size_t, c_uint64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libckv.so")

CKV_OK = 0
CKV_EINVAL = -1
CKV_ENOSPACE = -2
CKV_EHIP = -3
CKV_EUNSUPPORTED = -4


class CkvLayerStruct(Structure):
    """Mirror of ``ckv_layer`` (include/ckv.h); field order and types must match."""

    _fields_ = [
        ("batch", c_int32), ("n_kv_heads", c_int32), ("group", c_int32),
        ("head_dim", c_int32), ("n_sink", c_int32), ("n_clusters", c_int32),
        ("capacity", c_int32), ("n_total", c_int32), ("n_clustered", c_int32),
        ("n_pending", c_int32),
        ("k_tok", c_void_p), ("v_tok", c_void_p),
        ("k_clu", c_void_p), ("v_clu", c_void_p),
        ("k_clu_alt", c_void_p), ("v_clu_alt", c_void_p),
        ("cdir", c_void_p), ("csum", c_void_p), ("msum", c_void_p),
        ("cmean", c_void_p), ("csize", c_void_p), ("offsets", c_void_p),
        ("assign", c_void_p), ("perm", c_void_p),
        ("offsets_alt", c_void_p), ("cmean_alt", c_void_p),
    ]


class CkvError(RuntimeError):
    def __init__(self, func: str, code: int, message: str):
        super().__init__(f"{func} failed with code {code}: {message}")
        self.code = code
        self.message = message


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libckv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"libckv.so not found at {p}; build it with `python -m semantic_cluster_sparse_amd.build`")
    lib = ctypes.CDLL(p)
    LP = POINTER(CkvLayerStruct)
    lib.ckv_last_error.restype = c_char_p
    lib.ckv_last_error.argtypes = []
    lib.ckv_abi_layer_bytes.restype = c_size_t
    lib.ckv_abi_layer_bytes.argtypes = []
    lib.ckv_workspace_bytes.restype = c_size_t
    lib.ckv_workspace_bytes.argtypes = [LP, c_int32]
    lib.ckv_workspace_init.restype = c_int
    lib.ckv_workspace_init.argtypes = [c_void_p, c_size_t, c_void_p]
    lib.ckv_cluster_prefill.restype = c_int
    lib.ckv_cluster_prefill.argtypes = [LP, c_int32, c_int32, c_uint64, c_void_p, c_size_t, c_void_p]
    lib.ckv_cluster_prefill_indices.restype = c_int
    lib.ckv_cluster_prefill_indices.argtypes = [LP, c_int32, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.ckv_init_indices.restype = c_int
    lib.ckv_init_indices.argtypes = [LP, c_int32, c_uint64, c_void_p, c_void_p]
    lib.ckv_append.restype = c_int
    lib.ckv_append.argtypes = [LP, c_void_p, c_void_p, c_void_p]
    lib.ckv_cluster_incremental.restype = c_int
    lib.ckv_cluster_incremental.argtypes = [LP, c_void_p, c_size_t, c_void_p]
    lib.ckv_cluster_incremental_async.restype = c_int
    lib.ckv_cluster_incremental_async.argtypes = [LP, c_void_p, c_size_t, c_void_p]
    lib.ckv_cluster_commit.restype = c_int
    lib.ckv_cluster_commit.argtypes = [LP]
    lib.ckv_assign.restype = c_int
    lib.ckv_assign.argtypes = [LP, c_int32, c_void_p]
    lib.ckv_cluster_split.restype = c_int
    lib.ckv_cluster_split.argtypes = [LP, c_double, c_void_p, c_size_t, c_void_p]
    lib.ckv_select.restype = c_int
    lib.ckv_select.argtypes = [LP, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.ckv_append_select.restype = c_int
    lib.ckv_append_select.argtypes = [LP, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p]
    lib.ckv_workspace_bytes_per_head.restype = c_size_t
    lib.ckv_workspace_bytes_per_head.argtypes = [LP, c_int32]
    lib.ckv_select_per_head.restype = c_int
    lib.ckv_select_per_head.argtypes = [LP, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.ckv_sparse_decode_per_head.restype = c_int
    lib.ckv_sparse_decode_per_head.argtypes = [LP, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                               c_size_t, c_void_p]
    lib.ckv_sparse_decode.restype = c_int
    lib.ckv_sparse_decode.argtypes = [LP, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                      c_size_t, c_void_p]
    lib.ckv_select_decode.restype = c_int
    lib.ckv_select_decode.argtypes = [LP, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, LP, c_void_p, c_size_t,
                                      c_void_p]
    lib.ckv_append_select_decode.restype = c_int
    lib.ckv_append_select_decode.argtypes = [LP, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                             c_void_p, LP, c_void_p, c_size_t, c_void_p]
    lib.ckv_select_decode_per_head.restype = c_int
    lib.ckv_select_decode_per_head.argtypes = [LP, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, LP, c_void_p,
                                               c_size_t, c_void_p]
    lib.ckv_select_decode_noalloc_limit.restype = c_size_t
    lib.ckv_select_decode_noalloc_limit.argtypes = []
    lib.ckv_select_decode_noalloc.restype = c_int
    lib.ckv_select_decode_noalloc.argtypes = [LP, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, LP, c_void_p]
    if lib.ckv_abi_layer_bytes() != ctypes.sizeof(CkvLayerStruct):
        raise RuntimeError("ckv_layer layout mismatch between libckv.so and the binding")
    if path is None:
        _lib = lib
    return lib


def _check(func: str, rc: int) -> None:
    if rc != CKV_OK:
        raise CkvError(func, rc, ckv_last_error())


def _ref(layer):
    return ctypes.byref(layer)


def ckv_last_error() -> str:
    return load_library().ckv_last_error().decode(errors="replace")


def ckv_abi_layer_bytes() -> int:
    return int(load_library().ckv_abi_layer_bytes())


def ckv_workspace_bytes(layer: CkvLayerStruct, max_budget: int) -> int:
    n = int(load_library().ckv_workspace_bytes(_ref(layer), max_budget))
    if n == 0:
        raise CkvError("ckv_workspace_bytes", CKV_EINVAL, ckv_last_error())
    return n


def ckv_workspace_init(ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_workspace_init", load_library().ckv_workspace_init(ws, ws_bytes, stream))


def ckv_cluster_prefill(layer: CkvLayerStruct, n: int, iters: int, seed: int, ws: int,
                        ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_cluster_prefill",
           load_library().ckv_cluster_prefill(_ref(layer), n, iters, seed & (2 ** 64 - 1), ws, ws_bytes, stream))


def ckv_cluster_prefill_indices(layer: CkvLayerStruct, n: int, iters: int, init_idx: int, ws: int,
                                ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_cluster_prefill_indices",
           load_library().ckv_cluster_prefill_indices(_ref(layer), n, iters, init_idx, ws, ws_bytes, stream))


def ckv_init_indices(layer: CkvLayerStruct, n: int, seed: int, init_idx: int, stream: int = 0) -> None:
    _check("ckv_init_indices",
           load_library().ckv_init_indices(_ref(layer), n, seed & (2 ** 64 - 1), init_idx, stream))


def ckv_append(layer: CkvLayerStruct, k_new: int, v_new: int, stream: int = 0) -> None:
    _check("ckv_append", load_library().ckv_append(_ref(layer), k_new, v_new, stream))


def ckv_cluster_incremental(layer: CkvLayerStruct, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_cluster_incremental",
           load_library().ckv_cluster_incremental(_ref(layer), ws, ws_bytes, stream))


def ckv_cluster_incremental_async(layer: CkvLayerStruct, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_cluster_incremental_async",
           load_library().ckv_cluster_incremental_async(_ref(layer), ws, ws_bytes, stream))


def ckv_cluster_commit(layer: CkvLayerStruct) -> None:
    _check("ckv_cluster_commit", load_library().ckv_cluster_commit(_ref(layer)))


def ckv_assign(layer: CkvLayerStruct, n: int, stream: int = 0) -> None:
    _check("ckv_assign", load_library().ckv_assign(_ref(layer), n, stream))


def ckv_cluster_split(layer: CkvLayerStruct, threshold: float, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_cluster_split",
           load_library().ckv_cluster_split(_ref(layer), float(threshold), ws, ws_bytes, stream))


def ckv_select(layer: CkvLayerStruct, q: int, budget: int, sel_pos: int, sel_count: int, ws: int,
               ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_select",
           load_library().ckv_select(_ref(layer), q, budget, sel_pos, sel_count, ws, ws_bytes, stream))


def ckv_append_select(layer: CkvLayerStruct, k_new: int, v_new: int, q: int, budget: int, sel_pos: int,
                      sel_count: int, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_append_select",
           load_library().ckv_append_select(_ref(layer), k_new, v_new, q, budget, sel_pos, sel_count, ws,
                                            ws_bytes, stream))

def ckv_sparse_decode(layer: CkvLayerStruct, q: int, sel_pos: int, sel_count: int, budget: int,
                      out: int, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_sparse_decode",
           load_library().ckv_sparse_decode(_ref(layer), q, sel_pos, sel_count, budget, out, ws,
                                            ws_bytes, stream))


def ckv_workspace_bytes_per_head(layer: CkvLayerStruct, max_budget: int) -> int:
    n = int(load_library().ckv_workspace_bytes_per_head(_ref(layer), max_budget))
    if n == 0:
        raise CkvError("ckv_workspace_bytes_per_head", CKV_EINVAL, ckv_last_error())
    return n


def ckv_select_per_head(layer: CkvLayerStruct, q: int, budget: int, sel_pos: int, sel_count: int, ws: int,
                        ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_select_per_head",
           load_library().ckv_select_per_head(_ref(layer), q, budget, sel_pos, sel_count, ws, ws_bytes, stream))


def ckv_sparse_decode_per_head(layer: CkvLayerStruct, q: int, sel_pos: int, sel_count: int, budget: int,
                               out: int, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_sparse_decode_per_head",
           load_library().ckv_sparse_decode_per_head(_ref(layer), q, sel_pos, sel_count, budget, out, ws,
                                                     ws_bytes, stream))


def _opt_ref(layer):
    return ctypes.byref(layer) if layer is not None else None


def ckv_select_decode(layer: CkvLayerStruct, q: int, budget: int, sel_pos: int, sel_count: int, out: int,
                      next_layer, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_select_decode",
           load_library().ckv_select_decode(_ref(layer), q, budget, sel_pos, sel_count, out, _opt_ref(next_layer), ws,
                                            ws_bytes, stream))


def ckv_append_select_decode(layer: CkvLayerStruct, k_new: int, v_new: int, q: int, budget: int, sel_pos: int,
                             sel_count: int, out: int, next_layer, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_append_select_decode",
           load_library().ckv_append_select_decode(_ref(layer), k_new, v_new, q, budget, sel_pos, sel_count, out,
                                                   _opt_ref(next_layer), ws, ws_bytes, stream))


def ckv_select_decode_per_head(layer: CkvLayerStruct, q: int, budget: int, sel_pos: int, sel_count: int, out: int,
                               next_layer, ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check("ckv_select_decode_per_head",
           load_library().ckv_select_decode_per_head(_ref(layer), q, budget, sel_pos, sel_count, out,
                                                     _opt_ref(next_layer), ws, ws_bytes, stream))


def ckv_select_decode_noalloc_limit() -> int:
    return int(load_library().ckv_select_decode_noalloc_limit())


def ckv_select_decode_noalloc(layer: CkvLayerStruct, q: int, budget: int, sel_pos: int, sel_count: int, out: int,
                              next_layer=None, stream: int = 0) -> None:
    _check("ckv_select_decode_noalloc",
           load_library().ckv_select_decode_noalloc(_ref(layer), q, budget, sel_pos, sel_count, out,
                                                    _opt_ref(next_layer), stream))
