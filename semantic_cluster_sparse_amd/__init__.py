"""ClusterKV hot path on AMD Instinct MI355X (gfx950).

The compute lives in ``libckv.so`` (hand-written HIP, built in-tree by
``semantic_cluster_sparse_amd.build``).  ``ckv`` is a ctypes binding with the
same names as the C ABI in ``include/ckv.h``; ``layer.Layer`` allocates one
layer's device buffers with PyTorch and forwards to those calls.  There is no
CPU or PyTorch fallback: importing the binding fails loudly when the library
is missing.
"""

from .ckv import (  # noqa: F401
    CkvError,
    CkvLayerStruct,
    ckv_abi_layer_bytes,
    ckv_append,
    ckv_assign,
    ckv_append_select,
    ckv_append_select_decode,
    ckv_cluster_commit,
    ckv_cluster_incremental,
    ckv_cluster_incremental_async,
    ckv_cluster_prefill,
    ckv_cluster_prefill_indices,
    ckv_init_indices,
    ckv_cluster_split,
    ckv_last_error,
    ckv_select,
    ckv_select_decode,
    ckv_select_decode_noalloc,
    ckv_select_decode_noalloc_limit,
    ckv_select_decode_per_head,
    ckv_select_per_head,
    ckv_sparse_decode,
    ckv_sparse_decode_per_head,
    ckv_workspace_bytes,
    ckv_workspace_bytes_per_head,
    ckv_workspace_init,
    load_library,
    library_path,
)
