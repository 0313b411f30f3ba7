"""C-ABI boundary checks that need no GPU.

* libckv.so loads and exports every function include/ckv.h declares;
* the binding's mirror of ckv_layer has the library's size;
* argument errors come back as the documented codes before anything is
  enqueued (these calls never reach a HIP launch);
* workspace sizing is monotone in the sizes that drive it.
"""

import ctypes
import os
import re

import pytest

from semantic_cluster_sparse_amd import ckv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ckv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ckv.load_library()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_layer_struct_size_matches():
    assert ckv.ckv_abi_layer_bytes() == ctypes.sizeof(ckv.CkvLayerStruct)


def _layer(**kw):
    base = dict(batch=1, n_kv_heads=8, group=4, head_dim=128, n_sink=16, n_clusters=400,
                capacity=32768 + 64, n_total=0, n_clustered=0, n_pending=0)
    base.update(kw)
    return ckv.CkvLayerStruct(**base)


FAKE = 0x100000  # a 16-byte aligned non-null address; never dereferenced by these calls


def _fill_ptrs(L):
    for name, _ in ckv.CkvLayerStruct._fields_[10:]:
        setattr(L, name, FAKE)
    return L


def test_workspace_bytes_and_errors():
    L = _layer()
    n1 = ckv.ckv_workspace_bytes(L, 2048)
    assert n1 > 0 and n1 % 256 == 0
    assert ckv.ckv_workspace_bytes(_layer(batch=2), 2048) > n1
    assert ckv.ckv_workspace_bytes(_layer(capacity=65536), 2048) > n1
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_workspace_bytes(_layer(head_dim=64), 2048)
    assert "head_dim" in e.value.message
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_workspace_bytes(_layer(n_clusters=0), 2048)
    assert e.value.code == ckv.CKV_EINVAL


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, ckv.CKV_EUNSUPPORTED),
    ("group", 17, ckv.CKV_EUNSUPPORTED),
    ("group", 0, ckv.CKV_EINVAL),
    ("n_clusters", 2048, ckv.CKV_EUNSUPPORTED),
    ("n_sink", -1, ckv.CKV_EINVAL),
    ("capacity", 16, ckv.CKV_EINVAL),
])
def test_layer_validation(field, value, code):
    L = _fill_ptrs(_layer(**{field: value}))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_prefill(L, 32768, 10, 1234, FAKE, 1 << 40)
    assert e.value.code == code
    assert ckv.ckv_last_error()


def test_prefill_argument_errors():
    L = _fill_ptrs(_layer())
    cases = [
        (dict(n=32768, iters=0), ckv.CKV_EINVAL),               # no Lloyd round
        (dict(n=100, iters=10), ckv.CKV_EINVAL),                # K > m
        (dict(n=32768 + 65, iters=10), ckv.CKV_EINVAL),         # n > capacity
    ]
    for kw, code in cases:
        with pytest.raises(ckv.CkvError) as e:
            ckv.ckv_cluster_prefill(L, kw["n"], kw["iters"], 1234, FAKE, 1 << 40)
        with pytest.raises(ckv.CkvError) as e:
            ckv.ckv_cluster_prefill_indices(L, kw["n"], kw["iters"], FAKE, FAKE, 1 << 40)
        assert e.value.code == code, kw
        assert e.value.code == code, kw
    with pytest.raises(ckv.CkvError) as e:                      # misaligned init_idx
        ckv.ckv_cluster_prefill_indices(L, 32768, 10, FAKE + 4, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    with pytest.raises(ckv.CkvError) as e:                      # workspace too small
        ckv.ckv_cluster_prefill(L, 32768, 10, 1234, FAKE, 1024)
    assert e.value.code == ckv.CKV_ENOSPACE
    with pytest.raises(ckv.CkvError) as e:                      # no output for the drawn indices
        ckv.ckv_init_indices(L, 32768, 1234, None)
    assert e.value.code == ckv.CKV_EINVAL
    with pytest.raises(ckv.CkvError) as e:                      # K > m
        ckv.ckv_init_indices(L, 100, 1234, FAKE)
    assert e.value.code == ckv.CKV_EINVAL
    L.k_tok = None
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_prefill(L, 32768, 10, 1234, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    assert L.n_total == 0 and L.n_clustered == 0               # nothing advanced


def test_append_select_decode_errors():
    L = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=100, n_clustered=100))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_append(L, FAKE, FAKE)
    assert e.value.code == ckv.CKV_ENOSPACE and L.n_total == 100
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_select(L, FAKE, -1, FAKE, FAKE, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    L2 = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=20, n_clustered=20))
    with pytest.raises(ckv.CkvError) as e:                      # 4 clustered tokens < K
        ckv.ckv_select(L2, FAKE, 8, FAKE, FAKE, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    L3 = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=10, n_clustered=10))
    with pytest.raises(ckv.CkvError) as e:                      # n_clustered < n_sink
        ckv.ckv_sparse_decode(L3, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_sparse_decode(L, FAKE, FAKE, FAKE, 8, FAKE + 8, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_workspace_init(None, 16)
    assert e.value.code == ckv.CKV_EINVAL
    L4 = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=100, n_clustered=50))
    L4.k_clu_alt = None
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_incremental(L4, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL and L4.n_clustered == 50


def test_state_inconsistency_is_rejected():
    L = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=50, n_clustered=60))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_sparse_decode(L, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL


def test_async_incremental_and_commit_host_rules():
    # commit with nothing pending
    L = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_commit(L)
    assert e.value.code == ckv.CKV_EINVAL
    # the asynchronous form needs the second index and means
    L.offsets_alt = None
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_incremental_async(L, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL and L.n_pending == 0
    # no recent tokens: nothing to do, nothing pending
    L0 = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=100, n_clustered=100))
    ckv.ckv_cluster_incremental_async(L0, FAKE, 1 << 40)
    assert L0.n_pending == 0
    # while a result is pending, every other clustering call is refused
    P = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100, n_pending=120))
    for call in (lambda: ckv.ckv_cluster_incremental_async(P, FAKE, 1 << 40),
                 lambda: ckv.ckv_cluster_incremental(P, FAKE, 1 << 40),
                 lambda: ckv.ckv_cluster_prefill(P, 130, 2, 1234, FAKE, 1 << 40),
                 lambda: ckv.ckv_cluster_prefill_indices(P, 130, 2, FAKE, FAKE, 1 << 40)):
        with pytest.raises(ckv.CkvError) as e:
            call()
        assert e.value.code == ckv.CKV_EINVAL and "pending" in e.value.message
    # a pending count outside [n_clustered, n_total] is an inconsistent layer
    bad = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100, n_pending=140))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_commit(bad)
    assert e.value.code == ckv.CKV_EINVAL


def test_commit_swaps_the_second_buffers():
    L = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100, n_pending=120))
    names = ("k_clu", "v_clu", "offsets", "cmean")
    for i, n in enumerate(names):
        setattr(L, n, FAKE + 0x1000 * (2 * i + 1))
        setattr(L, n + "_alt", FAKE + 0x1000 * (2 * i + 2))
    before = {n: (getattr(L, n), getattr(L, n + "_alt")) for n in names}
    ckv.ckv_cluster_commit(L)
    for n in names:
        assert (getattr(L, n), getattr(L, n + "_alt")) == before[n][::-1], n
    assert L.n_clustered == 120 and L.n_pending == 0 and L.n_total == 130


def test_split_host_rules():
    L = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_split(L, float("nan"), FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL and "NaN" in e.value.message
    P = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100, n_pending=120))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_split(P, 0.5, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL and "pending" in e.value.message
    N = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=10, n_clustered=10))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_split(N, 0.5, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL and "no cluster state" in e.value.message
    L.assign = None
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_cluster_split(L, 0.5, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    S = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100))
    with pytest.raises(ckv.CkvError):
        ckv.ckv_cluster_split(S, 0.5, FAKE, 64)            # workspace too small
    # nothing clustered beyond the sinks: nothing to do, nothing enqueued
    E = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=16, n_clustered=16))
    ckv.ckv_cluster_split(E, 0.5, FAKE, 1 << 40)
    assert E.n_clustered == 16 and E.n_total == 16


def test_assign_host_rules():
    L = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100))
    for n, what in ((201, "capacity"), (16, "n_sink"), (3, "n_sink")):
        with pytest.raises(ckv.CkvError) as e:
            ckv.ckv_assign(L, n)
        assert e.value.code == ckv.CKV_EINVAL and what in e.value.message
    P = _fill_ptrs(_layer(capacity=200, n_clusters=8, n_total=130, n_clustered=100, n_pending=120))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_assign(P, 100)
    assert e.value.code == ckv.CKV_EINVAL and "pending" in e.value.message
    L.cdir = None
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_assign(L, 100)
    assert e.value.code == ckv.CKV_EINVAL and "cdir" in e.value.message


def test_select_decode_host_rules():
    L = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=100, n_clustered=100))
    with pytest.raises(ckv.CkvError) as e:                      # full cache: nothing appended
        ckv.ckv_append_select_decode(L, FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, None, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_ENOSPACE and L.n_total == 100
    for call in (ckv.ckv_select_decode, ckv.ckv_select_decode_per_head):
        with pytest.raises(ckv.CkvError) as e:
            call(L, FAKE, -1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40)
        assert e.value.code == ckv.CKV_EINVAL
        with pytest.raises(ckv.CkvError) as e:                  # output not 16-byte aligned
            call(L, FAKE, 8, FAKE, FAKE, FAKE + 4, None, FAKE, 1 << 40)
        assert e.value.code == ckv.CKV_EINVAL
        with pytest.raises(ckv.CkvError) as e:                  # workspace too small
            call(L, FAKE, 8, FAKE, FAKE, FAKE, L, FAKE, 256)
        assert e.value.code == ckv.CKV_ENOSPACE
    L2 = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=20, n_clustered=20))
    with pytest.raises(ckv.CkvError) as e:                      # 4 clustered tokens < K
        ckv.ckv_select_decode(L2, FAKE, 8, FAKE, FAKE, FAKE, None, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_append_select_decode(L2, None, FAKE, FAKE, 8, FAKE, FAKE, FAKE, None, FAKE, 1 << 40)
    assert e.value.code == ckv.CKV_EINVAL and L2.n_total == 20
    # the fused call needs the decode's partials and the recall's cut scores at once
    L3 = _layer()
    assert ckv.ckv_workspace_bytes_per_head(L3, 2048) >= ckv.ckv_workspace_bytes(L3, 2048)


def test_select_decode_noalloc_host_rules():
    assert ckv.ckv_select_decode_noalloc_limit() == 16 << 20
    # the cut-score area alone (64 units x 131056 rows x 4 B) is beyond the limit: refused before any launch
    big = _fill_ptrs(_layer(batch=64, n_kv_heads=1, capacity=131072, n_total=131072, n_clustered=131072))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_select_decode_noalloc(big, FAKE, 2048, FAKE, FAKE, FAKE)
    assert e.value.code == ckv.CKV_ENOSPACE and "limit" in e.value.message
    L = _fill_ptrs(_layer(capacity=100, n_clusters=8, n_total=100, n_clustered=100))
    with pytest.raises(ckv.CkvError) as e:
        ckv.ckv_select_decode_noalloc(L, FAKE, -1, FAKE, FAKE, FAKE)
    assert e.value.code == ckv.CKV_EINVAL


def test_missing_library_fails_loudly(tmp_path):
    # the binding has no fallback: without the built library every call path raises
    with pytest.raises(RuntimeError, match="libckv.so not found"):
        ckv.load_library(str(tmp_path / "libckv.so"))
