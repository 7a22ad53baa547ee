"""H2O chunked sparse attention on MI355X: Python binding of libh2o.

Argument marshalling only: every step runs in the HIP kernels of
``csrc/`` behind the C ABI of ``include/h2o.h``.  PyTorch supplies device
memory and streams.  Layouts and semantics are those of the C header.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._native import (  # noqa: F401
    H2O_BF16, H2O_ERR_CAPACITY, H2O_ERR_HIP, H2O_ERR_INVALID_ARG, H2O_ERR_UNSUPPORTED,
    H2O_ERR_WORKSPACE, H2O_F32, H2O_OK, H2O_SCORE_H2O, H2O_SCORE_H2O_NORM, KERNEL_IDS,
    LIB_PATH, CacheStruct, Dims, H2OError, check, lib,
)

SCORE_MODES = {"h2o": H2O_SCORE_H2O, "h2o_norm": H2O_SCORE_H2O_NORM}
_TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}
_C_DTYPES = {"bf16": H2O_BF16, "f32": H2O_F32}


@dataclass(frozen=True)
class H2ODims:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    recent_window: int
    dtype: str = "bf16"          # "bf16" | "f32"

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]

    def c(self) -> Dims:
        return Dims(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.capacity,
                    self.recent_window, _C_DTYPES[self.dtype])


class H2OCache:
    """One layer's cache: device tensors k, v [B,Hkv,N_C,d], pos int32 and score fp32
    [B,Hkv,N_C], plus the host-side count of filled slots and the next position."""

    def __init__(self, dims: H2ODims, device="cuda"):
        B, Hkv, NC, d = dims.batch, dims.n_kv_heads, dims.capacity, dims.head_dim
        self.dims = dims
        self.k = torch.zeros(B, Hkv, NC, d, dtype=dims.torch_dtype, device=device)
        self.v = torch.zeros(B, Hkv, NC, d, dtype=dims.torch_dtype, device=device)
        self.pos = torch.full((B, Hkv, NC), -1, dtype=torch.int32, device=device)
        self.score = torch.zeros(B, Hkv, NC, dtype=torch.float32, device=device)
        self.n_valid = 0
        self.next_pos = 0

    def reset(self):
        self.n_valid = 0
        self.next_pos = 0

    def load(self, k, v, pos, score, n_valid, next_pos):
        self.k.copy_(k)
        self.v.copy_(v)
        self.pos.copy_(pos)
        self.score.copy_(score)
        self.n_valid = int(n_valid)
        self.next_pos = int(next_pos)

    def c(self) -> CacheStruct:
        return CacheStruct(self.k.data_ptr(), self.v.data_ptr(), self.pos.data_ptr(),
                           self.score.data_ptr(), self.n_valid)


def _stream_ptr(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, shape, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def workspace_bytes(dims: H2ODims, chunk_len: int) -> int:
    return int(lib.h2o_workspace_bytes(ctypes.byref(dims.c()), chunk_len))


def chunk_attn(cache: H2OCache, chunk_start: int, q, k_new, v_new, sm_scale: float,
               out=None, lse=None, colsum_cache=None, colsum_new=None, workspace=None,
               stream=None, summed_weights=True):
    """h2o_chunk_attn: returns (out, lse, colsum_cache, colsum_new).  With
    ``summed_weights=False`` both colsum buffers are NULL (returned as None)."""
    d = cache.dims
    B, Hq, Hkv, D, NC = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.capacity
    S = q.shape[2]
    dev = cache.k.device
    _need(q, (B, Hq, S, D), d.torch_dtype, "q")
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    if out is None:
        out = torch.empty(B, Hq, S, D, dtype=d.torch_dtype, device=dev)
    if lse is None:
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
    _need(out, (B, Hq, S, D), d.torch_dtype, "out")
    _need(lse, (B, Hq, S), torch.float32, "lse")
    if summed_weights:
        if colsum_cache is None:
            colsum_cache = torch.empty(B, Hkv, NC, dtype=torch.float32, device=dev)
        if colsum_new is None:
            colsum_new = torch.empty(B, Hkv, S, dtype=torch.float32, device=dev)
        _need(colsum_cache, (B, Hkv, NC), torch.float32, "colsum_cache")
        _need(colsum_new, (B, Hkv, S), torch.float32, "colsum_new")
        cs_ptrs = (colsum_cache.data_ptr(), colsum_new.data_ptr())
    else:
        colsum_cache = colsum_new = None
        cs_ptrs = (None, None)
    ws_need = workspace_bytes(d, S)
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib.h2o_chunk_attn(ctypes.byref(d.c()), ctypes.byref(cache.c()), int(chunk_start), S,
                             float(sm_scale), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                             out.data_ptr(), lse.data_ptr(), cs_ptrs[0], cs_ptrs[1],
                             ws_ptr, ws_len, _stream_ptr(stream, dev)))
    return out, lse, colsum_cache, colsum_new


def chunk_attn_noalloc(cache: H2OCache, chunk_start: int, q, k_new, v_new, sm_scale: float,
                       out, lse, colsum_cache=None, colsum_new=None, stream=None):
    """h2o_chunk_attn_noalloc: h2o_chunk_attn with the library's static device scratch as
    workspace (the library allocates nothing; the caller passes every output).  Both colsum
    buffers None: no summed weights.  Returns (out, lse, colsum_cache, colsum_new)."""
    d = cache.dims
    B, Hq, Hkv, D, NC = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.capacity
    S = q.shape[2]
    _need(q, (B, Hq, S, D), d.torch_dtype, "q")
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    _need(out, (B, Hq, S, D), d.torch_dtype, "out")
    _need(lse, (B, Hq, S), torch.float32, "lse")
    if (colsum_cache is None) != (colsum_new is None):
        raise ValueError("colsum_cache and colsum_new: both or neither")
    cs_ptrs = (None, None)
    if colsum_cache is not None:
        _need(colsum_cache, (B, Hkv, NC), torch.float32, "colsum_cache")
        _need(colsum_new, (B, Hkv, S), torch.float32, "colsum_new")
        cs_ptrs = (colsum_cache.data_ptr(), colsum_new.data_ptr())
    check(lib.h2o_chunk_attn_noalloc(ctypes.byref(d.c()), ctypes.byref(cache.c()),
                                     int(chunk_start), S, float(sm_scale), q.data_ptr(),
                                     k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), cs_ptrs[0], cs_ptrs[1],
                                     _stream_ptr(stream, cache.k.device)))
    return out, lse, colsum_cache, colsum_new


def update_scores(cache: H2OCache, colsum_cache, stream=None):
    """h2o_update_scores: cache.score[..., :n_valid] += colsum_cache[..., :n_valid]."""
    d = cache.dims
    _need(colsum_cache, (d.batch, d.n_kv_heads, d.capacity), torch.float32, "colsum_cache")
    check(lib.h2o_update_scores(ctypes.byref(d.c()), ctypes.byref(cache.c()),
                                colsum_cache.data_ptr(), _stream_ptr(stream, cache.k.device)))


def evict_and_insert(cache: H2OCache, chunk_start: int, k_new, v_new, colsum_new,
                     freed_slots=None, score_mode="h2o", stream=None):
    """h2o_evict_and_insert: returns freed_slots [B,Hkv,S] and advances cache.n_valid."""
    d = cache.dims
    B, Hkv, D = d.batch, d.n_kv_heads, d.head_dim
    S = k_new.shape[2]
    dev = cache.k.device
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    _need(colsum_new, (B, Hkv, S), torch.float32, "colsum_new")
    if freed_slots is None:
        freed_slots = torch.empty(B, Hkv, S, dtype=torch.int32, device=dev)
    _need(freed_slots, (B, Hkv, S), torch.int32, "freed_slots")
    cs = cache.c()
    check(lib.h2o_evict_and_insert(ctypes.byref(d.c()), ctypes.byref(cs), int(chunk_start), S,
                                   SCORE_MODES[score_mode], k_new.data_ptr(), v_new.data_ptr(),
                                   colsum_new.data_ptr(), freed_slots.data_ptr(), None, 0,
                                   _stream_ptr(stream, dev)))
    cache.n_valid = cs.n_valid
    cache.next_pos = int(chunk_start) + S
    return freed_slots


def update_evict_and_insert(cache: H2OCache, chunk_start: int, colsum_cache, k_new, v_new,
                            colsum_new, freed_slots=None, score_mode="h2o", stream=None):
    """h2o_update_evict_and_insert: update_scores then evict_and_insert in one call (the
    update runs inside the selection when slots are evicted); returns freed_slots."""
    d = cache.dims
    B, Hkv, D = d.batch, d.n_kv_heads, d.head_dim
    S = k_new.shape[2]
    dev = cache.k.device
    _need(colsum_cache, (B, Hkv, d.capacity), torch.float32, "colsum_cache")
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    _need(colsum_new, (B, Hkv, S), torch.float32, "colsum_new")
    if freed_slots is None:
        freed_slots = torch.empty(B, Hkv, S, dtype=torch.int32, device=dev)
    _need(freed_slots, (B, Hkv, S), torch.int32, "freed_slots")
    cs = cache.c()
    check(lib.h2o_update_evict_and_insert(ctypes.byref(d.c()), ctypes.byref(cs),
                                          colsum_cache.data_ptr(), int(chunk_start), S,
                                          SCORE_MODES[score_mode], k_new.data_ptr(),
                                          v_new.data_ptr(), colsum_new.data_ptr(),
                                          freed_slots.data_ptr(), _stream_ptr(stream, dev)))
    cache.n_valid = cs.n_valid
    cache.next_pos = int(chunk_start) + S
    return freed_slots


def chunk_step(cache: H2OCache, chunk_start: int, q, k_new, v_new, sm_scale: float,
               score_mode="h2o", out=None, lse=None, colsum_cache=None, colsum_new=None,
               freed_slots=None, workspace=None, stream=None):
    """h2o_chunk_step: the whole chunk (attention with summed weights, score update,
    eviction, insertion); returns (out, lse, colsum_cache, colsum_new, freed_slots) and
    advances cache.n_valid / cache.next_pos."""
    d = cache.dims
    B, Hq, Hkv, D, NC = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.capacity
    S = q.shape[2]
    dev = cache.k.device
    _need(q, (B, Hq, S, D), d.torch_dtype, "q")
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    out = torch.empty(B, Hq, S, D, dtype=d.torch_dtype, device=dev) if out is None else out
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev) if lse is None else lse
    if colsum_cache is None:
        colsum_cache = torch.empty(B, Hkv, NC, dtype=torch.float32, device=dev)
    if colsum_new is None:
        colsum_new = torch.empty(B, Hkv, S, dtype=torch.float32, device=dev)
    if freed_slots is None:
        freed_slots = torch.empty(B, Hkv, S, dtype=torch.int32, device=dev)
    _need(out, (B, Hq, S, D), d.torch_dtype, "out")
    _need(lse, (B, Hq, S), torch.float32, "lse")
    _need(colsum_cache, (B, Hkv, NC), torch.float32, "colsum_cache")
    _need(colsum_new, (B, Hkv, S), torch.float32, "colsum_new")
    _need(freed_slots, (B, Hkv, S), torch.int32, "freed_slots")
    ws_need = workspace_bytes(d, S)
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    cs = cache.c()
    check(lib.h2o_chunk_step(ctypes.byref(d.c()), ctypes.byref(cs), int(chunk_start), S,
                             float(sm_scale), SCORE_MODES[score_mode], q.data_ptr(),
                             k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             colsum_cache.data_ptr(), colsum_new.data_ptr(),
                             freed_slots.data_ptr(), ws_ptr, ws_len, _stream_ptr(stream, dev)))
    cache.n_valid = cs.n_valid
    cache.next_pos = int(chunk_start) + S
    return out, lse, colsum_cache, colsum_new, freed_slots


def select_slots(cache: H2OCache, chunk_start: int, chunk_len: int, freed_slots=None,
                 score_mode="h2o", stream=None):
    """h2o_select_slots: the chunk's targets [B,Hkv,S] from the current scores; the cache
    is not modified."""
    d = cache.dims
    dev = cache.k.device
    if freed_slots is None:
        freed_slots = torch.empty(d.batch, d.n_kv_heads, chunk_len, dtype=torch.int32,
                                  device=dev)
    _need(freed_slots, (d.batch, d.n_kv_heads, chunk_len), torch.int32, "freed_slots")
    check(lib.h2o_select_slots(ctypes.byref(d.c()), ctypes.byref(cache.c()), int(chunk_start),
                               int(chunk_len), SCORE_MODES[score_mode], freed_slots.data_ptr(),
                               _stream_ptr(stream, dev)))
    return freed_slots


def buffer_attn(cache: H2OCache, chunk_start: int, q, k_new, v_new, freed_slots,
                sm_scale: float, out=None, lse=None, colsum_cache=None, colsum_new=None,
                workspace=None, stream=None, summed_weights=True):
    """h2o_buffer_attn: returns (out, lse, colsum_cache, colsum_new); the targets below
    n_valid in freed_slots are not keys."""
    d = cache.dims
    B, Hq, Hkv, D, NC = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.capacity
    S = q.shape[2]
    dev = cache.k.device
    _need(q, (B, Hq, S, D), d.torch_dtype, "q")
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    _need(freed_slots, (B, Hkv, S), torch.int32, "freed_slots")
    if out is None:
        out = torch.empty(B, Hq, S, D, dtype=d.torch_dtype, device=dev)
    if lse is None:
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
    _need(out, (B, Hq, S, D), d.torch_dtype, "out")
    _need(lse, (B, Hq, S), torch.float32, "lse")
    if summed_weights:
        if colsum_cache is None:
            colsum_cache = torch.empty(B, Hkv, NC, dtype=torch.float32, device=dev)
        if colsum_new is None:
            colsum_new = torch.empty(B, Hkv, S, dtype=torch.float32, device=dev)
        _need(colsum_cache, (B, Hkv, NC), torch.float32, "colsum_cache")
        _need(colsum_new, (B, Hkv, S), torch.float32, "colsum_new")
        cs_ptrs = (colsum_cache.data_ptr(), colsum_new.data_ptr())
    else:
        colsum_cache = colsum_new = None
        cs_ptrs = (None, None)
    ws_need = workspace_bytes(d, S)
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib.h2o_buffer_attn(ctypes.byref(d.c()), ctypes.byref(cache.c()), int(chunk_start), S,
                              float(sm_scale), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                              freed_slots.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              cs_ptrs[0], cs_ptrs[1], ws_ptr, ws_len, _stream_ptr(stream, dev)))
    return out, lse, colsum_cache, colsum_new


def insert(cache: H2OCache, chunk_start: int, k_new, v_new, freed_slots, colsum_new=None,
           stream=None):
    """h2o_insert: chunk token i into freed_slots[..., i] (score colsum_new, or 0)."""
    d = cache.dims
    B, Hkv, D = d.batch, d.n_kv_heads, d.head_dim
    S = k_new.shape[2]
    dev = cache.k.device
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    _need(freed_slots, (B, Hkv, S), torch.int32, "freed_slots")
    if colsum_new is not None:
        _need(colsum_new, (B, Hkv, S), torch.float32, "colsum_new")
    cs = cache.c()
    check(lib.h2o_insert(ctypes.byref(d.c()), ctypes.byref(cs), int(chunk_start), S,
                         k_new.data_ptr(), v_new.data_ptr(),
                         colsum_new.data_ptr() if colsum_new is not None else None,
                         freed_slots.data_ptr(), _stream_ptr(stream, dev)))
    cache.n_valid = cs.n_valid
    cache.next_pos = int(chunk_start) + S


def chunk_attn_backward(cache: H2OCache, chunk_start: int, q, k_new, v_new, out, lse, dout,
                        sm_scale: float, freed_slots=None, grads=None, workspace=None,
                        stream=None):
    """h2o_chunk_attn_backward: returns (dq, dk_new, dv_new, dk_cache, dv_cache), float32.
    The cache must be as it stood for the forward call that produced out and lse."""
    d = cache.dims
    B, Hq, Hkv, D, NC = d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim, d.capacity
    S = q.shape[2]
    dev = cache.k.device
    _need(q, (B, Hq, S, D), d.torch_dtype, "q")
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    _need(out, (B, Hq, S, D), d.torch_dtype, "out")
    _need(lse, (B, Hq, S), torch.float32, "lse")
    _need(dout, (B, Hq, S, D), d.torch_dtype, "dout")
    if freed_slots is not None:
        _need(freed_slots, (B, Hkv, S), torch.int32, "freed_slots")
    g = grads or {}
    shapes = {"dq": (B, Hq, S, D), "dk_new": (B, Hkv, S, D), "dv_new": (B, Hkv, S, D),
              "dk_cache": (B, Hkv, NC, D), "dv_cache": (B, Hkv, NC, D)}
    res = []
    for name, shape in shapes.items():
        t = g.get(name)
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=dev)
        _need(t, shape, torch.float32, name)
        res.append(t)
    ws_need = int(lib.h2o_backward_workspace_bytes(ctypes.byref(d.c()), S))
    if workspace is None:
        workspace = torch.empty(max(1, ws_need), dtype=torch.uint8, device=dev)
    check(lib.h2o_chunk_attn_backward(
        ctypes.byref(d.c()), ctypes.byref(cache.c()), int(chunk_start), S, float(sm_scale),
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), out.data_ptr(), lse.data_ptr(),
        dout.data_ptr(), freed_slots.data_ptr() if freed_slots is not None else None,
        *[t.data_ptr() for t in res], workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev)))
    return tuple(res)


def evict_and_insert_lastrec(cache: H2OCache, chunk_start: int, k_new, v_new, sink_tokens: int,
                             freed_slots=None, stream=None):
    """h2o_evict_and_insert_lastrec: returns freed_slots [B,Hkv,S], advances cache.n_valid."""
    d = cache.dims
    B, Hkv, D = d.batch, d.n_kv_heads, d.head_dim
    S = k_new.shape[2]
    dev = cache.k.device
    _need(k_new, (B, Hkv, S, D), d.torch_dtype, "k_new")
    _need(v_new, (B, Hkv, S, D), d.torch_dtype, "v_new")
    if freed_slots is None:
        freed_slots = torch.empty(B, Hkv, S, dtype=torch.int32, device=dev)
    _need(freed_slots, (B, Hkv, S), torch.int32, "freed_slots")
    cs = cache.c()
    check(lib.h2o_evict_and_insert_lastrec(ctypes.byref(d.c()), ctypes.byref(cs), int(chunk_start),
                                           S, int(sink_tokens), k_new.data_ptr(),
                                           v_new.data_ptr(), freed_slots.data_ptr(),
                                           _stream_ptr(stream, dev)))
    cache.n_valid = cs.n_valid
    cache.next_pos = int(chunk_start) + S
    return freed_slots


def step(cache: H2OCache, q, k_new, v_new, sm_scale: float, score_mode="h2o", bufs=None,
         stream=None, policy="h2o", sink_tokens=0):
    """One chunk at position cache.next_pos.  policy "h2o": one h2o_chunk_step call
    (attention with summed weights, score update, eviction by ``score_mode``, insertion).
    policy "h2o_buffer": the insert-first buffer
    form (targets from the scores before the chunk, attention over the buffer, score
    update, insertion).  policy "lastrec": attention alone, then eviction by position
    keeping the first ``sink_tokens``.  ``bufs`` (a dict holding out, lse, colsum_cache,
    colsum_new, freed_slots, workspace) is reused if given."""
    b = bufs or {}
    P = cache.next_pos
    if policy == "h2o_buffer":
        S = q.shape[2]
        freed = select_slots(cache, P, S, b.get("freed_slots"), score_mode, stream)
        out, lse, cs_cache, cs_new = buffer_attn(cache, P, q, k_new, v_new, freed, sm_scale,
                                                 b.get("out"), b.get("lse"),
                                                 b.get("colsum_cache"), b.get("colsum_new"),
                                                 b.get("workspace"), stream)
        update_scores(cache, cs_cache, stream)
        insert(cache, P, k_new, v_new, freed, cs_new, stream)
        return {"out": out, "lse": lse, "colsum_cache": cs_cache, "colsum_new": cs_new,
                "freed_slots": freed}
    if policy == "lastrec":
        out, lse, _, _ = chunk_attn(cache, P, q, k_new, v_new, sm_scale, b.get("out"),
                                    b.get("lse"), workspace=b.get("workspace"), stream=stream,
                                    summed_weights=False)
        freed = evict_and_insert_lastrec(cache, P, k_new, v_new, sink_tokens,
                                         b.get("freed_slots"), stream)
        return {"out": out, "lse": lse, "freed_slots": freed}
    if policy != "h2o":
        raise ValueError(f"unknown policy {policy!r}")
    out, lse, cs_cache, cs_new, freed = chunk_step(
        cache, P, q, k_new, v_new, sm_scale, score_mode, b.get("out"), b.get("lse"),
        b.get("colsum_cache"), b.get("colsum_new"), b.get("freed_slots"), b.get("workspace"),
        stream)
    return {"out": out, "lse": lse, "colsum_cache": cs_cache, "colsum_new": cs_new,
            "freed_slots": freed}


class KernelTimer:
    """Sum of per-launch durations of one library kernel, from HIP events the library
    records on the launch stream (h2o_kernel_timer_start / _stop)."""

    def __init__(self, kernel: str, max_launches: int = 65536):
        self.kid = KERNEL_IDS[kernel]
        self.max = max_launches
        self.total_ms = 0.0
        self.launches = 0

    def __enter__(self):
        check(lib.h2o_kernel_timer_start(self.kid, self.max))
        return self

    def __exit__(self, *exc):
        ms = ctypes.c_double()
        cnt = ctypes.c_int64()
        check(lib.h2o_kernel_timer_stop(self.kid, ctypes.byref(ms), ctypes.byref(cnt)))
        self.total_ms, self.launches = ms.value, cnt.value
        return False

    @property
    def mean_ms(self) -> float:
        return self.total_ms / max(1, self.launches)
