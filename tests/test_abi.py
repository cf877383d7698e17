"""The C-ABI library loads and exports every entry point its header declares;
host-side argument checks answer without touching a GPU."""
import ctypes as C
import os
import re

import pytest

from context_packed_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cp_attn.h")


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_attn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for s in ("cp_attn_rank_metadata", "cp_attn_fwd", "cp_attn_bwd"):
        assert s in syms
    assert set(syms) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for s in declared_symbols():
        assert hasattr(lib, s), s


def test_host_argument_checks_without_gpu():
    lib = _lib.load()
    h = C.c_void_p()
    assert lib.cp_attn_rank_metadata(None, None, 1, 2, 0, -1, 16, None, C.byref(h)) == _lib.ERR_INVALID_ARG
    assert b"cu_seqlens" in lib.cp_attn_last_error()
    dummy = C.c_void_p(16)
    assert lib.cp_attn_rank_metadata(dummy, None, 0, 2, 0, -1, 16, None, C.byref(h)) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_rank_metadata(dummy, None, 1, 17, 0, -1, 16, None, C.byref(h)) == _lib.ERR_UNSUPPORTED
    assert lib.cp_attn_rank_metadata(dummy, None, 1, 4, 4, -1, 16, None, C.byref(h)) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_rank_metadata(dummy, None, 1, 4, 1, 2, 16, None, C.byref(h)) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_fwd(None, None, None, None, 1, 1, 128, 1.0, 1, None, None, None, 0, None) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_bwd(None, None, None, None, None, None, None, 1, 1, 128, 1.0, 1, None, None, None, None, 0,
                           None) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_workspace_bytes(None, 1, 1, 128, 0) == 0
    lib.cp_attn_meta_free(None)
    g = C.c_void_p()
    assert lib.cp_attn_graph_capture(None, 3, None, None, None, 1, 1, 128, 1.0, 1, None, None, None, None, None,
                                     None, None, 0, None, 0, C.byref(g)) == _lib.ERR_INVALID_ARG
    assert not g.value
    assert lib.cp_attn_graph_capture(dummy, 3, None, None, None, 1, 1, 128, 1.0, 1, None, None, None, None, None,
                                     None, None, 0, None, 0, None) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_graph_launch(None, None) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_graph_kernels(None) == 0
    lib.cp_attn_graph_free(None)
    assert lib.cp_attn_a2a_seq_to_head(None, 2, 0, 4, 256, None, None, None) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_a2a_head_to_seq(None, 2, 0, 4, 256, None, None, None) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_ag_workspace_bytes(None, 1, 1, 128, 0) == 0
    ms, tf = C.c_double(), C.c_double()
    assert lib.cp_attn_mfma_probe(0, dummy, None, C.byref(ms), C.byref(tf)) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_mfma_probe(10, None, None, C.byref(ms), C.byref(tf)) == _lib.ERR_INVALID_ARG
    assert lib.cp_attn_ag_fwd(None, None, None, None, 1, 1, 128, 1.0, 1, None, None, None, 0, None) == \
        _lib.ERR_INVALID_ARG
    assert lib.cp_attn_ag_bwd(None, None, None, None, None, None, None, 1, 1, 128, 1.0, 1, None, None, None, None, 0,
                              None) == _lib.ERR_INVALID_ARG
