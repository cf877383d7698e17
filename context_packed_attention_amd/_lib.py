"""ctypes loader for libcpattn.so: prototypes of every symbol in include/cp_attn.h."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcpattn.so")

MAX_CP = 16

# status codes
OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 2
ERR_HINT_MISMATCH = 3
ERR_WORKSPACE = 4
ERR_HIP = 5
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "HINT_MISMATCH", 4: "WORKSPACE", 5: "HIP"}

EXPORTED = [
    "cp_attn_rank_metadata", "cp_attn_rank_metadata_host", "cp_attn_meta_summary", "cp_attn_meta_export", "cp_attn_meta_free",
    "cp_attn_workspace_bytes", "cp_attn_fwd", "cp_attn_bwd", "cp_attn_bwd_noalloc", "cp_attn_shard_gather", "cp_attn_last_error",
    "cp_attn_timing_enable", "cp_attn_timing_read",
    "cp_attn_graph_capture", "cp_attn_graph_launch", "cp_attn_graph_kernels", "cp_attn_graph_free",
    "cp_attn_a2a_seq_to_head", "cp_attn_a2a_head_to_seq",
    "cp_attn_ag_workspace_bytes", "cp_attn_ag_fwd", "cp_attn_ag_bwd", "cp_attn_mfma_probe",
]


class Summary(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("cp_size", C.c_int32), ("cp_rank", C.c_int32),
        ("pad_between_seqs", C.c_int32), ("t_local", C.c_int32), ("has_tail", C.c_int32),
        ("t_alloc", C.c_int64),
        ("step_kind", C.c_int32 * MAX_CP), ("step_src", C.c_int32 * MAX_CP),
        ("tiles_fwd", C.c_int64 * MAX_CP), ("tiles_dkdv", C.c_int64 * MAX_CP),
        ("valid_rows", C.c_int64),
    ]


_lib = None


def load(path: str | None = None) -> C.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libcpattn.so not built ({p}); build it with python -m context_packed_attention_amd.build")
    lib = C.CDLL(p)
    vp = C.c_void_p
    i32 = C.c_int32
    st = C.c_int
    lib.cp_attn_rank_metadata.argtypes = [vp, vp, i32, i32, i32, i32, C.c_int64, vp, C.POINTER(vp)]
    lib.cp_attn_rank_metadata.restype = st
    lib.cp_attn_rank_metadata_host.argtypes = [vp, vp, i32, i32, i32, i32, C.c_int64, vp, C.POINTER(vp)]
    lib.cp_attn_rank_metadata_host.restype = st
    lib.cp_attn_meta_summary.argtypes = [vp, C.POINTER(Summary)]
    lib.cp_attn_meta_summary.restype = st
    lib.cp_attn_meta_export.argtypes = [vp, C.POINTER(C.c_int32), C.c_size_t, C.POINTER(C.c_size_t)]
    lib.cp_attn_meta_export.restype = st
    lib.cp_attn_meta_free.argtypes = [vp]
    lib.cp_attn_meta_free.restype = None
    lib.cp_attn_workspace_bytes.argtypes = [vp, i32, i32, i32, i32]
    lib.cp_attn_workspace_bytes.restype = C.c_size_t
    lib.cp_attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, C.c_float, i32, vp, vp, vp, C.c_size_t, vp]
    lib.cp_attn_fwd.restype = st
    lib.cp_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, C.c_float, i32, vp, vp, vp, vp,
                                C.c_size_t, vp]
    lib.cp_attn_bwd.restype = st
    lib.cp_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, C.c_float, i32, vp, vp, vp, vp]
    lib.cp_attn_bwd_noalloc.restype = st
    lib.cp_attn_shard_gather.argtypes = [vp, i32, vp, vp, C.c_size_t, vp]
    lib.cp_attn_shard_gather.restype = st
    lib.cp_attn_timing_enable.argtypes = [i32]
    lib.cp_attn_timing_enable.restype = st
    lib.cp_attn_timing_read.argtypes = [C.c_char_p, i32, C.POINTER(C.c_double), C.POINTER(C.c_int64), i32]
    lib.cp_attn_timing_read.restype = i32
    lib.cp_attn_graph_capture.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, C.c_float, i32, vp, vp, vp, vp, vp,
                                          vp, vp, C.c_size_t, vp, C.c_size_t, C.POINTER(vp)]
    lib.cp_attn_graph_capture.restype = st
    lib.cp_attn_graph_launch.argtypes = [vp, vp]
    lib.cp_attn_graph_launch.restype = st
    lib.cp_attn_graph_kernels.argtypes = [vp]
    lib.cp_attn_graph_kernels.restype = C.c_int64
    lib.cp_attn_graph_free.argtypes = [vp]
    lib.cp_attn_graph_free.restype = None
    for f in (lib.cp_attn_a2a_seq_to_head, lib.cp_attn_a2a_head_to_seq):
        f.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
        f.restype = st
    lib.cp_attn_ag_workspace_bytes.argtypes = [vp, i32, i32, i32, i32]
    lib.cp_attn_ag_workspace_bytes.restype = C.c_size_t
    lib.cp_attn_ag_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, C.c_float, i32, vp, vp, vp, C.c_size_t, vp]
    lib.cp_attn_ag_fwd.restype = st
    lib.cp_attn_ag_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, C.c_float, i32, vp, vp, vp, vp,
                                   C.c_size_t, vp]
    lib.cp_attn_ag_bwd.restype = st
    lib.cp_attn_mfma_probe.argtypes = [i32, vp, vp, C.POINTER(C.c_double), C.POINTER(C.c_double)]
    lib.cp_attn_mfma_probe.restype = st
    lib.cp_attn_last_error.argtypes = []
    lib.cp_attn_last_error.restype = C.c_char_p
    _lib = lib
    return lib
