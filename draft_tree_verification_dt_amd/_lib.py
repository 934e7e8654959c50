"""ctypes declarations of libdtree's C ABI (include/dtree.h).

The shared library is loaded from this package's directory. There is no
fallback: if it is missing, loading raises and nothing else runs.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdtree.so")

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_p = ctypes.c_void_p
c_size = ctypes.c_size_t
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)
P_f32 = ctypes.POINTER(ctypes.c_float)
P_f64 = ctypes.POINTER(ctypes.c_double)

DT_OK = 0
DT_ERR_NULL = -1
DT_ERR_SHAPE = -2
DT_ERR_TREE = -3
DT_ERR_VALUE = -4
DT_ERR_UNSUPPORTED = -5
DT_ERR_WORKSPACE = -6
DT_ERR_HIP = -7
DT_ERR_NOMEM = -8
DT_MAX_TREE_NODES = 1024


class dt_attn_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", c_i32),
        ("num_q_heads", c_i32),
        ("num_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("softmax_scale", ctypes.c_float),
        ("split_keys", c_i32),
        ("node_offsets", P_i32),
        ("prefix_lens", P_i32),
        ("prefix_row_start", P_i64),
        ("q_row_stride", c_i64),
        ("out_row_stride", c_i64),
        ("tree_row_stride", c_i64),
        ("prefix_row_stride", c_i64),
        ("prefix_head_stride", c_i64),
        ("phase_stamps", ctypes.c_void_p),
        ("phase_stamp_rows", c_i64),
    ]


class dt_commit_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", c_i32),
        ("num_layers", c_i32),
        ("num_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("max_path", c_i32),
        ("node_offsets", P_i32),
        ("prefix_lens", P_i32),
        ("prefix_row_start", P_i64),
        ("cache_rows", P_i64),
        ("tree_row_stride", c_i64),
        ("cache_row_stride", c_i64),
        ("cache_head_stride", c_i64),
    ]


P_vp = ctypes.POINTER(ctypes.c_void_p)

# name -> (restype, argtypes)
SIGNATURES = {
    "dt_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dt_abi_version": (ctypes.c_int, []),
    "dt_build_tree": (ctypes.c_int, [c_i32, c_i32, P_f32, P_i32, c_i32, c_i32, P_i32, P_i32, P_i32, P_f64, P_i32]),
    "dt_validate_tree": (ctypes.c_int, [P_i32, c_i32]),
    "dt_tree_attention_workspace_size": (ctypes.c_int, [ctypes.POINTER(dt_attn_desc), ctypes.POINTER(c_size)]),
    "dt_tree_attention": (ctypes.c_int, [ctypes.POINTER(dt_attn_desc), c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_size, c_p]),
    "dt_tree_attention_noalloc": (ctypes.c_int, [ctypes.POINTER(dt_attn_desc), c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    "dt_argmax_rows_workspace_size": (ctypes.c_int, [c_i64, c_i64, ctypes.POINTER(c_size)]),
    "dt_argmax_rows": (ctypes.c_int, [c_p, c_i64, c_i64, c_i64, c_p, c_p, c_size, c_p]),
    "dt_sample_rows_workspace_size": (ctypes.c_int, [c_i64, c_i64, ctypes.POINTER(c_size)]),
    "dt_sample_rows": (ctypes.c_int, [c_p, c_i64, c_i64, c_i64, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, c_p,
                                      c_p, c_size, c_p]),
    "dt_accept_path": (ctypes.c_int, [c_i32, P_i32, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    "dt_commit_kv": (ctypes.c_int, [ctypes.POINTER(dt_commit_desc), P_vp, P_vp, P_vp, P_vp, c_p, c_p, c_p]),
    "dt_topk_rows_workspace_size": (ctypes.c_int, [c_i64, c_i64, c_i32, ctypes.POINTER(c_size)]),
    "dt_topk_rows": (ctypes.c_int, [c_p, c_i64, c_i64, c_i64, c_i32, c_p, c_p, c_p, c_size, c_p]),
    "dt_expand_depth": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, ctypes.c_float, c_p, c_i64, c_p, c_i64, c_p, c_i64,
                                       c_p, c_p, c_p, c_p, c_i64, c_p]),
    "dt_prune_topb": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
}

_lib = None


def load():
    """Load libdtree.so (once) and declare every entry point."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime under the same soname as ROCm's;
        # whichever is loaded first serves the whole process. Load torch's
        # first so that libdtree and the tensors it is handed share one runtime.
        import torch  # noqa: F401

        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m draft_tree_verification_dt_amd.build`"
                "; there is no fallback implementation")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
