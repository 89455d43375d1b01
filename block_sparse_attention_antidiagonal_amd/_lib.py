"""ctypes view of libbsa.so: the C ABI declared in include/bsa.h, nothing more.

Loading fails loudly when the library has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; BSA_LIB_PATH may name another build of the same library.
LIB_PATH = os.environ.get("BSA_LIB_PATH") or os.path.join(_HERE, "libbsa.so")

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_size_p = ctypes.POINTER(ctypes.c_size_t)

# name -> argument types (every call returns int status unless listed in _RESTYPES)
SIGNATURES = {
    "bsa_status_string": [c_int],
    "bsa_abi_version": [],
    "bsa_cluster_layout_workspace_size": [c_int, c_int, c_int, c_size_p],
    "bsa_cluster_layout": [c_int, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_select_probe_rows_layouts": [c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
    "bsa_centroids": [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                      c_void_p, c_void_p],
    "bsa_antidiag_scores_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_antidiag_scores": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int,
                            c_float, c_int, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_antidiag_scores_heads": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int,
                                  c_int, c_float, c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_pooled_qk_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_pooled_qk": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p, c_void_p,
                      c_void_p, c_size_t, c_void_p],
    "bsa_mask_reuse_decide": [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_float, c_int,
                              c_int, c_void_p, c_void_p, c_void_p],
    "bsa_mask_reuse_update": [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
    "bsa_top_p_mask": [c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p],
    "bsa_mask_lists": [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p],
    "bsa_kv_pack_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_kv_pack": [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_void_p,
                    c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_sparse_attention_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_sparse_attention": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_float, c_void_p, c_void_p, c_int,
                             c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_int,
                             c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_sparse_attention_static_scratch_bytes": [],
    "bsa_sparse_attention_noalloc": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_float, c_void_p, c_void_p,
                                     c_int, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                     c_size_t, c_int, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p],
    "bsa_response_partition_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_response_partition": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_float, c_int, c_int,
                               c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                               c_void_p],
    "bsa_kmeans_workspace_size": [c_int, c_int, c_int, c_size_p],
    "bsa_kmeans": [c_int, c_int, c_int, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_kv_pack_centroids": [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                              c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_probe_attention_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_probe_attention": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_float,
                            c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_probe_attention_packed_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_probe_attention_packed": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_float, c_void_p, c_int,
                                   c_void_p, c_size_t, c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, c_int, c_int,
                                   c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_probe_fit": [c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int, c_float, c_int, c_void_p,
                      c_void_p, c_void_p],
    "bsa_query_centroids": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int,
                            c_void_p, c_void_p],
    "bsa_block_error_workspace_size": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_size_p],
    "bsa_block_error": [c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_int, c_float, c_void_p, c_size_t,
                        c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "bsa_error_route": [c_void_p, c_int, c_int, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p],
    "bsa_probe_apply": [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p],
    "bsa_correct": [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
    "bsa_gather_rows": [c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p, c_void_p],
    "bsa_select_probe_rows": [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p],
    "bsa_tile_labels": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p],
    "bsa_sliding_tile_mask": [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p],
}
_RESTYPES = {"bsa_status_string": ctypes.c_char_p, "bsa_sparse_attention_static_scratch_bytes": ctypes.c_size_t}

BSA_F32, BSA_BF16 = 0, 1
MAX_FIT_PROBES = 65536  # bsa_probe_fit: 2 <= M <= this
MAX_PROBE_ROWS = 1024  # bsa_probe_attention(_packed): M <= this


class BsaError(RuntimeError):
    def __init__(self, name: str, status: int, text: str):
        super().__init__(f"{name} failed with status {status}: {text}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libbsa.so (once) and declare every exported call."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its HIP runtime must be the one libbsa.so binds to (loading the library
    # first would bring in a second runtime whose launches fail).
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python block_sparse_attention_antidiagonal_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, c_int)
    _lib = lib
    return lib


def call(name: str, *args) -> None:
    """Call an ABI function and raise BsaError on a non-zero status."""
    lib = load()
    status = getattr(lib, name)(*args)
    if status != 0:
        raise BsaError(name, status, lib.bsa_status_string(status).decode())


def size_query(name: str, *args) -> int:
    out = ctypes.c_size_t(0)
    call(name, *args, ctypes.byref(out))
    return int(out.value)
