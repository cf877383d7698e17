"""Python binding of the C ABI (argument marshalling only).

Every function forwards to the entry point of the same name in libcpattn.so
(include/cp_attn.h). PyTorch only provides device memory (``data_ptr``) and
the current stream; all work runs in the library's HIP kernels. There is no
fallback: if the library is missing these functions raise.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib as L


class CpAttnError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {L.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(rc: int, where: str):
    if rc != L.OK:
        msg = L.load().cp_attn_last_error().decode(errors="replace")
        raise CpAttnError(rc, where, msg)


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _need(t, name: str, nbytes: int, dtype: str | None = None):
    """Layout checks the C ABI cannot make (it sees only pointers): a torch
    tensor argument must be a contiguous device tensor of the right element
    type holding at least `nbytes`. Raw integer pointers pass unchecked."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: a device tensor is required")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and str(t.dtype) != "torch." + dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected torch.{dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: holds {have} bytes, the call needs {nbytes}")


def _need_list(ts, name: str, count: int, nbytes: int, dtype: str | None = None):
    if len(ts) != count:
        raise ValueError(f"{name}: {len(ts)} tensors given, cp_size is {count}")
    for i, t in enumerate(ts):
        _need(t, f"{name}[{i}]", nbytes, dtype)


def _ptr_array(ts):
    arr = (C.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


class Meta:
    """Owns a cp_attn_meta handle (freed on close / garbage collection)."""

    def __init__(self, handle: int, t_alloc: int = 0):
        self._h = C.c_void_p(handle)
        self.t_alloc = int(t_alloc)  # rows of the rank's local tensors
        s = L.Summary()
        _check(L.load().cp_attn_meta_summary(self._h, C.byref(s)), "cp_attn_meta_summary")
        self.summary = s

    @property
    def handle(self):
        if not self._h:
            raise ValueError("metadata handle already freed")
        return self._h

    @property
    def t_local(self) -> int:
        return int(self.summary.t_local)

    @property
    def cp(self) -> int:
        return int(self.summary.cp_size)

    @property
    def t_global(self) -> int:
        """Rows of the whole packed batch, cu_seqlens_padded[B]."""
        return self.t_local * self.cp

    def steps(self):
        s = self.summary
        return [(int(s.step_kind[i]), int(s.step_src[i])) for i in range(s.cp_size)]

    def export(self) -> np.ndarray:
        return cp_attn_meta_export(self)

    def close(self):
        if self._h:
            L.load().cp_attn_meta_free(self._h)
            self._h = C.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cp_attn_rank_metadata(cu_seqlens, cu_seqlens_padded, cp_size: int, cp_rank: int, pad_hint: int = -1,
                          t_alloc: int | None = None, stream=None, B: int | None = None) -> Meta:
    """cu_seqlens / cu_seqlens_padded: device int32 tensors [B+1] (padded may be
    the same tensor, a distinct copy, or None)."""
    if B is None:
        B = cu_seqlens.numel() - 1
    if t_alloc is None:
        raise ValueError("t_alloc is required")
    h = C.c_void_p()
    rc = L.load().cp_attn_rank_metadata(_ptr(cu_seqlens), _ptr(cu_seqlens_padded), int(B), int(cp_size),
                                        int(cp_rank), int(pad_hint), int(t_alloc), _stream(stream), C.byref(h))
    _check(rc, "cp_attn_rank_metadata")
    return Meta(h.value, int(t_alloc))


def cp_attn_rank_metadata_host(cu_seqlens, cu_seqlens_padded, cp_size: int, cp_rank: int, pad_hint: int = -1,
                               t_alloc: int | None = None, stream=None) -> Meta:
    """The same handle from HOST int32 sequences [B+1] (numpy arrays or lists;
    padded may be None), with no synchronisation."""
    if t_alloc is None:
        raise ValueError("t_alloc is required")
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    cup = None if cu_seqlens_padded is None else np.ascontiguousarray(cu_seqlens_padded, dtype=np.int32)
    if cu.ndim != 1 or cu.size < 2 or (cup is not None and cup.shape != cu.shape):
        raise ValueError("cu_seqlens / cu_seqlens_padded must be 1-D of the same length >= 2")
    h = C.c_void_p()
    rc = L.load().cp_attn_rank_metadata_host(cu.ctypes.data_as(C.c_void_p),
                                             None if cup is None else cup.ctypes.data_as(C.c_void_p),
                                             int(cu.size - 1), int(cp_size), int(cp_rank), int(pad_hint),
                                             int(t_alloc), _stream(stream), C.byref(h))
    _check(rc, "cp_attn_rank_metadata_host")
    return Meta(h.value, int(t_alloc))


def cp_attn_meta_export(meta: Meta) -> np.ndarray:
    lib = L.load()
    n = C.c_size_t()
    _check(lib.cp_attn_meta_export(meta.handle, None, 0, C.byref(n)), "cp_attn_meta_export")
    buf = (C.c_int32 * n.value)()
    _check(lib.cp_attn_meta_export(meta.handle, buf, n.value, C.byref(n)), "cp_attn_meta_export")
    return np.frombuffer(buf, dtype=np.int32).copy()


def cp_attn_workspace_bytes(meta: Meta, hq: int, hkv: int, d: int, pass_: int) -> int:
    return int(L.load().cp_attn_workspace_bytes(meta.handle, hq, hkv, d, pass_))


def _check_fwd(meta: Meta, q, k_shards, v_shards, hq, hkv, d, out, lse):
    ta = meta.t_alloc
    _need(q, "q", ta * hq * d * 2, "bfloat16")
    _need_list(k_shards, "k_shards", meta.cp, ta * hkv * d * 2, "bfloat16")
    _need_list(v_shards, "v_shards", meta.cp, ta * hkv * d * 2, "bfloat16")
    _need(out, "out", ta * hq * d * 2, "bfloat16")
    _need(lse, "lse", hq * ta * 4, "float32")


def _check_bwd(meta: Meta, hq, hkv, d, dout, dq, dk_parts, dv_parts):
    ta = meta.t_alloc
    _need(dout, "dout", ta * hq * d * 2, "bfloat16")
    _need(dq, "dq", ta * hq * d * 2, "bfloat16")
    _need_list(dk_parts, "dk_parts", meta.cp, ta * hkv * d * 2, "bfloat16")
    _need_list(dv_parts, "dv_parts", meta.cp, ta * hkv * d * 2, "bfloat16")


def cp_attn_fwd(meta: Meta, q, k_shards, v_shards, hq: int, hkv: int, d: int, softmax_scale: float,
                causal: int, out, lse, workspace, stream=None):
    _check_fwd(meta, q, k_shards, v_shards, hq, hkv, d, out, lse)
    ks = _ptr_array(k_shards)
    vs = _ptr_array(v_shards)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = L.load().cp_attn_fwd(meta.handle, _ptr(q), ks, vs, hq, hkv, d, float(softmax_scale), int(causal),
                              _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "cp_attn_fwd")


def cp_attn_bwd(meta: Meta, q, k_shards, v_shards, out, lse, dout, hq: int, hkv: int, d: int,
                softmax_scale: float, causal: int, dq, dk_parts, dv_parts, workspace, stream=None):
    _check_fwd(meta, q, k_shards, v_shards, hq, hkv, d, out, lse)
    _check_bwd(meta, hq, hkv, d, dout, dq, dk_parts, dv_parts)
    ks = _ptr_array(k_shards)
    vs = _ptr_array(v_shards)
    dks = _ptr_array(dk_parts)
    dvs = _ptr_array(dv_parts)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = L.load().cp_attn_bwd(meta.handle, _ptr(q), ks, vs, _ptr(out), _ptr(lse), _ptr(dout), hq, hkv, d,
                              float(softmax_scale), int(causal), _ptr(dq), dks, dvs, _ptr(workspace), ws_bytes,
                              _stream(stream))
    _check(rc, "cp_attn_bwd")


def cp_attn_bwd_noalloc(meta: Meta, q, k_shards, v_shards, out, lse, dout, hq: int, hkv: int, d: int,
                        softmax_scale: float, causal: int, dq, dk_parts, dv_parts, stream=None):
    """cp_attn_bwd with no workspace: the library's fixed scratch array."""
    _check_fwd(meta, q, k_shards, v_shards, hq, hkv, d, out, lse)
    _check_bwd(meta, hq, hkv, d, dout, dq, dk_parts, dv_parts)
    rc = L.load().cp_attn_bwd_noalloc(meta.handle, _ptr(q), _ptr_array(k_shards), _ptr_array(v_shards), _ptr(out),
                                      _ptr(lse), _ptr(dout), hq, hkv, d, float(softmax_scale), int(causal), _ptr(dq),
                                      _ptr_array(dk_parts), _ptr_array(dv_parts), _stream(stream))
    _check(rc, "cp_attn_bwd_noalloc")


def cp_attn_shard_gather(meta: Meta, shard: int, global_rows, local_rows, row_bytes: int, stream=None):
    _need(global_rows, "global_rows", meta.t_global * row_bytes)
    _need(local_rows, "local_rows", meta.t_local * row_bytes)
    rc = L.load().cp_attn_shard_gather(meta.handle, int(shard), _ptr(global_rows), _ptr(local_rows),
                                       int(row_bytes), _stream(stream))
    _check(rc, "cp_attn_shard_gather")


def cp_attn_last_error() -> str:
    return L.load().cp_attn_last_error().decode(errors="replace")


def cp_attn_timing_enable(on: bool):
    _check(L.load().cp_attn_timing_enable(1 if on else 0), "cp_attn_timing_enable")


def cp_attn_mfma_probe(iters: int, sink, stream=None) -> tuple:
    """(ms, TFLOP/s) of one launch of the library's matrix-unit calibration
    kernel; sink: a device float32 tensor of at least one element."""
    import torch
    if not isinstance(sink, torch.Tensor) or not sink.is_cuda or sink.dtype != torch.float32 or sink.numel() < 1:
        raise ValueError("sink must be a float32 CUDA tensor of at least one element")
    ms, tf = C.c_double(), C.c_double()
    rc = L.load().cp_attn_mfma_probe(int(iters), sink.data_ptr(), _stream(stream), C.byref(ms), C.byref(tf))
    _check(rc, "cp_attn_mfma_probe")
    return float(ms.value), float(tf.value)


def cp_attn_timing_read(max_kernels: int = 32) -> dict:
    """{kernel name: (total ms, launches)} of the launches recorded since enabling."""
    name_len = 64
    names = C.create_string_buffer(max_kernels * name_len)
    ms = (C.c_double * max_kernels)()
    cnt = (C.c_int64 * max_kernels)()
    n = L.load().cp_attn_timing_read(names, name_len, ms, cnt, max_kernels)
    if n < 0:
        raise CpAttnError(L.ERR_HIP, "cp_attn_timing_read", "event synchronisation failed")
    raw = names.raw
    out = {}
    for i in range(n):
        nm = raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (float(ms[i]), int(cnt[i]))
    return out


def meta_tables(meta: Meta) -> dict:
    """The exported integer tables as named lists (layout of cp_attn_meta_export)."""
    a = [int(x) for x in cp_attn_meta_export(meta)]
    B, cp, rank, pad, tl, tail, nst = a[:7]
    o = 8
    out = {"B": B, "cp": cp, "rank": rank, "pad_between_seqs": pad, "t_local": tl, "has_tail": tail}

    def take(n):
        nonlocal o
        v = a[o:o + n]
        o += n
        return v

    out["chunk"] = take(B)
    out["cu_padded_local"] = take(B + 1)
    out["cu_padded_half"] = take(B + 1)
    for s in range(cp):
        for k in ("full", "first", "second"):
            out[f"cu_{k}_{s}"] = take(B + 1)
    out["steps"] = []
    for _ in range(nst):
        kind, src = take(2)
        out["steps"].append({"kind": kind, "src": src, "q_start": take(B), "q_len": take(B),
                             "kv_start": take(B), "kv_len": take(B)})
    return out


def step_pairs(meta: Meta) -> list[int]:
    """Causal (query, key) pairs each ring step computes, diagonal included:
    n(n+1)/2 per sequence at the causal step, q_len * kv_len otherwise."""
    t = meta_tables(meta)
    pairs = []
    for st in t["steps"]:
        if st["kind"] == 0:
            pairs.append(sum(n * (n + 1) // 2 for n in st["q_len"]))
        else:
            pairs.append(sum(a * b for a, b in zip(st["q_len"], st["kv_len"])))
    return pairs


class Graph:
    """Owns a cp_attn_graph: one rank share's forward and/or backward captured
    as a HIP graph (freed on close / garbage collection). The tensors it was
    captured with must outlive it; replays read their current contents."""

    def __init__(self, handle: int, keep):
        self._h = C.c_void_p(handle)
        self._keep = keep  # the captured buffers stay referenced while the graph lives

    @property
    def kernels(self) -> int:
        return int(L.load().cp_attn_graph_kernels(self._h))

    def launch(self, stream=None):
        if not self._h:
            raise ValueError("graph already freed")
        _check(L.load().cp_attn_graph_launch(self._h, _stream(stream)), "cp_attn_graph_launch")

    def close(self):
        if self._h:
            L.load().cp_attn_graph_free(self._h)
            self._h = C.c_void_p(None)
            self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cp_attn_graph_capture(meta: Meta, passes: int, q, k_shards, v_shards, hq: int, hkv: int, d: int,
                          softmax_scale: float, causal: int, out, lse, dout=None, dq=None, dk_parts=(),
                          dv_parts=(), ws_fwd=None, ws_bwd=None) -> Graph:
    _check_fwd(meta, q, k_shards, v_shards, hq, hkv, d, out, lse)
    if int(passes) & 2:
        _check_bwd(meta, hq, hkv, d, dout, dq, dk_parts, dv_parts)
    ks = _ptr_array(k_shards)
    vs = _ptr_array(v_shards)
    dks = _ptr_array(dk_parts) if dk_parts else None
    dvs = _ptr_array(dv_parts) if dv_parts else None
    wf = ws_fwd.numel() * ws_fwd.element_size() if ws_fwd is not None else 0
    wb = ws_bwd.numel() * ws_bwd.element_size() if ws_bwd is not None else 0
    h = C.c_void_p()
    rc = L.load().cp_attn_graph_capture(meta.handle, int(passes), _ptr(q), ks, vs, hq, hkv, d, float(softmax_scale),
                                        int(causal), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), dks, dvs,
                                        _ptr(ws_fwd), wf, _ptr(ws_bwd), wb, C.byref(h))
    _check(rc, "cp_attn_graph_capture")
    keep = (meta, q, tuple(k_shards), tuple(v_shards), out, lse, dout, dq, tuple(dk_parts), tuple(dv_parts),
            ws_fwd, ws_bwd)
    return Graph(h.value, keep)


def cp_attn_a2a_seq_to_head(meta: Meta, a2a_size: int, p2p_rank: int, heads: int, head_bytes: int, ins, outs,
                            stream=None):
    """Group p2p_rank's all-to-all: ins[a] = CP rank p*A + a's local tensor
    (all heads), outs[a'] = head group a' of p2p rank p's local rows."""
    _need_list(ins, "ins", a2a_size, meta.t_local * heads * head_bytes)
    _need_list(outs, "outs", a2a_size, meta.t_local * heads * head_bytes)
    rc = L.load().cp_attn_a2a_seq_to_head(meta.handle, int(a2a_size), int(p2p_rank), int(heads), int(head_bytes),
                                          _ptr_array(ins), _ptr_array(outs), _stream(stream))
    _check(rc, "cp_attn_a2a_seq_to_head")


def cp_attn_a2a_head_to_seq(meta: Meta, a2a_size: int, p2p_rank: int, heads: int, head_bytes: int, ins, outs,
                            stream=None):
    """The inverse all-to-all: ins[a'] = head group a' of p2p rank p's local
    rows, outs[a] = CP rank p*A + a's local tensor (all heads)."""
    _need_list(ins, "ins", a2a_size, meta.t_local * heads * head_bytes)
    _need_list(outs, "outs", a2a_size, meta.t_local * heads * head_bytes)
    rc = L.load().cp_attn_a2a_head_to_seq(meta.handle, int(a2a_size), int(p2p_rank), int(heads), int(head_bytes),
                                          _ptr_array(ins), _ptr_array(outs), _stream(stream))
    _check(rc, "cp_attn_a2a_head_to_seq")


def cp_attn_ag_workspace_bytes(meta: Meta, hq: int, hkv: int, d: int, pass_: int) -> int:
    return int(L.load().cp_attn_ag_workspace_bytes(meta.handle, hq, hkv, d, pass_))


def cp_attn_ag_fwd(meta: Meta, q, k_full, v_full, hq: int, hkv: int, d: int, softmax_scale: float, causal: int,
                   out, lse, workspace, stream=None):
    """All-gather share, forward: k_full / v_full are the gathered K / V in
    packed (cu_seqlens_padded) order."""
    ta = meta.t_alloc
    _need(q, "q", ta * hq * d * 2, "bfloat16")
    _need(k_full, "k_full", meta.t_global * hkv * d * 2, "bfloat16")
    _need(v_full, "v_full", meta.t_global * hkv * d * 2, "bfloat16")
    _need(out, "out", ta * hq * d * 2, "bfloat16")
    _need(lse, "lse", hq * ta * 4, "float32")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = L.load().cp_attn_ag_fwd(meta.handle, _ptr(q), _ptr(k_full), _ptr(v_full), hq, hkv, d, float(softmax_scale),
                                 int(causal), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "cp_attn_ag_fwd")


def cp_attn_ag_bwd(meta: Meta, q, k_full, v_full, out, lse, dout, hq: int, hkv: int, d: int, softmax_scale: float,
                   causal: int, dq, dk_full, dv_full, workspace, stream=None):
    """All-gather share, backward: dk_full / dv_full receive this rank's
    contribution to every gathered key row."""
    ta = meta.t_alloc
    for t, nm in ((q, "q"), (out, "out"), (dout, "dout"), (dq, "dq")):
        _need(t, nm, ta * hq * d * 2, "bfloat16")
    for t, nm in ((k_full, "k_full"), (v_full, "v_full"), (dk_full, "dk_full"), (dv_full, "dv_full")):
        _need(t, nm, meta.t_global * hkv * d * 2, "bfloat16")
    _need(lse, "lse", hq * ta * 4, "float32")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = L.load().cp_attn_ag_bwd(meta.handle, _ptr(q), _ptr(k_full), _ptr(v_full), _ptr(out), _ptr(lse), _ptr(dout),
                                 hq, hkv, d, float(softmax_scale), int(causal), _ptr(dq), _ptr(dk_full),
                                 _ptr(dv_full), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "cp_attn_ag_bwd")
