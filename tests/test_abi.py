"""The C-ABI library loads, exports what include/h2o.h declares, and rejects bad
arguments on the host before anything is launched (CPU only: no call here reaches
a kernel)."""
import ctypes
import os
import re

import pytest

import h2o_sparse_attention_amd as h2o
from h2o_sparse_attention_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h2o.h")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"H2O_API\s+[\w\s\*]+?\b(h2o_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("h2o_chunk_attn", "h2o_update_scores", "h2o_evict_and_insert",
                     "h2o_workspace_bytes", "h2o_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_native.LIB_PATH)
    names = declared_functions()
    assert names, "no declarations found"
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_native._SIGNATURES), "binding and header disagree"


def test_abi_version():
    assert h2o.lib.h2o_abi_version() == 1


def _dims(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64, capacity=256,
                recent_window=32, dtype=_native.H2O_BF16)
    base.update(kw)
    return _native.Dims(**base)


FAKE = 0x1000   # never dereferenced: every call below must fail validation first


def _attn(dims, n_valid=0, S=64, P=0, scale=0.125, q=FAKE, ws=None, wsb=0, cache_ptrs=FAKE):
    cache = _native.CacheStruct(cache_ptrs, cache_ptrs, cache_ptrs, cache_ptrs, n_valid)
    return h2o.lib.h2o_chunk_attn(ctypes.byref(dims), ctypes.byref(cache), P, S, scale, q, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=4, n_kv_heads=3), _native.H2O_ERR_INVALID_ARG),
    (dict(batch=0), _native.H2O_ERR_INVALID_ARG),
    (dict(n_kv_heads=0), _native.H2O_ERR_INVALID_ARG),
    (dict(head_dim=96), _native.H2O_ERR_UNSUPPORTED),
    (dict(head_dim=256), _native.H2O_ERR_UNSUPPORTED),
    (dict(dtype=7), _native.H2O_ERR_UNSUPPORTED),
    (dict(capacity=0), _native.H2O_ERR_UNSUPPORTED),
    (dict(capacity=32769), _native.H2O_ERR_UNSUPPORTED),
    (dict(recent_window=-1), _native.H2O_ERR_INVALID_ARG),
])
def test_chunk_attn_rejects_bad_dims(kw, status):
    assert _attn(_dims(**kw)) == status
    assert h2o.lib.h2o_last_error().decode()


@pytest.mark.parametrize("call,status", [
    (dict(n_valid=-1), _native.H2O_ERR_INVALID_ARG),
    (dict(n_valid=257), _native.H2O_ERR_INVALID_ARG),
    (dict(S=0), _native.H2O_ERR_INVALID_ARG),
    (dict(P=-5), _native.H2O_ERR_INVALID_ARG),
    (dict(P=2**31 - 10), _native.H2O_ERR_UNSUPPORTED),
    (dict(scale=0.0), _native.H2O_ERR_INVALID_ARG),
    (dict(scale=-1.0), _native.H2O_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _native.H2O_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _native.H2O_ERR_INVALID_ARG),
    (dict(q=None), _native.H2O_ERR_INVALID_ARG),
    (dict(cache_ptrs=None), _native.H2O_ERR_INVALID_ARG),
])
def test_chunk_attn_rejects_bad_call(call, status):
    assert _attn(_dims(), **call) == status
    assert h2o.lib.h2o_last_error().decode()


def test_null_dims_and_cache():
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, 0)
    st = h2o.lib.h2o_chunk_attn(None, ctypes.byref(cache), 0, 1, 1.0, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, None, 0, None)
    assert st == _native.H2O_ERR_INVALID_ARG
    d = _dims()
    st = h2o.lib.h2o_chunk_attn(ctypes.byref(d), None, 0, 1, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, None, 0, None)
    assert st == _native.H2O_ERR_INVALID_ARG
    assert h2o.lib.h2o_update_scores(ctypes.byref(d), ctypes.byref(cache), None, None) == \
        _native.H2O_ERR_INVALID_ARG


def _evict(dims, n_valid, S, P=1000, mode=0, freed=FAKE):
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, n_valid)
    st = h2o.lib.h2o_evict_and_insert(ctypes.byref(dims), ctypes.byref(cache), P, S, mode, FAKE,
                                      FAKE, FAKE, freed, None, 0, None)
    return st, cache.n_valid


def test_evict_capacity_rule():
    # full cache, S + W > N_C: some chunk could find too few eligible slots
    st, n = _evict(_dims(capacity=256, recent_window=200), n_valid=256, S=64)
    assert st == _native.H2O_ERR_CAPACITY and n == 256
    assert "capacity" in h2o.lib.h2o_last_error().decode()
    # chunk longer than the cache
    st, _ = _evict(_dims(capacity=32, recent_window=0), n_valid=0, S=64)
    assert st == _native.H2O_ERR_CAPACITY


def test_evict_rejects_bad_args():
    assert _evict(_dims(), 10, 8, mode=5)[0] == _native.H2O_ERR_INVALID_ARG
    assert _evict(_dims(), 10, 8, freed=None)[0] == _native.H2O_ERR_INVALID_ARG
    assert _evict(_dims(), 10, 0)[0] == _native.H2O_ERR_INVALID_ARG
    assert _evict(_dims(head_dim=32), 10, 8)[0] == _native.H2O_ERR_UNSUPPORTED


def _update_evict(dims, n_valid, S, P=1000, mode=0, cs=FAKE, freed=FAKE):
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, n_valid)
    st = h2o.lib.h2o_update_evict_and_insert(ctypes.byref(dims), ctypes.byref(cache), cs, P, S,
                                             mode, FAKE, FAKE, FAKE, freed, None)
    return st, cache.n_valid


def test_update_evict_rejects_before_launching():
    """The fused update + eviction call validates exactly like the two calls: every error is
    returned before any launch, the cache count untouched."""
    st, n = _update_evict(_dims(capacity=256, recent_window=200), n_valid=256, S=64)
    assert st == _native.H2O_ERR_CAPACITY and n == 256
    assert _update_evict(_dims(), 10, 8, cs=None)[0] == _native.H2O_ERR_INVALID_ARG
    assert "colsum_cache" in h2o.lib.h2o_last_error().decode()
    assert _update_evict(_dims(), 10, 8, mode=5)[0] == _native.H2O_ERR_INVALID_ARG
    assert _update_evict(_dims(), 10, 8, freed=None)[0] == _native.H2O_ERR_INVALID_ARG
    assert _update_evict(_dims(), 10, 0)[0] == _native.H2O_ERR_INVALID_ARG
    assert _update_evict(_dims(head_dim=32), 10, 8)[0] == _native.H2O_ERR_UNSUPPORTED


def _lastrec(dims, n_valid, S, sink, P=1000, freed=FAKE):
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, n_valid)
    st = h2o.lib.h2o_evict_and_insert_lastrec(ctypes.byref(dims), ctypes.byref(cache), P, S,
                                              sink, FAKE, FAKE, freed, None)
    return st, cache.n_valid


def test_lastrec_capacity_rule():
    # full cache, S + beta > N_C: the first beta positions may leave too few eligible slots
    st, n = _lastrec(_dims(capacity=256, recent_window=0), n_valid=256, S=64, sink=200)
    assert st == _native.H2O_ERR_CAPACITY and n == 256
    assert "sink_tokens" in h2o.lib.h2o_last_error().decode()
    # the recent window plays no part in lastrec: S + W > N_C alone is not refused here
    # (the call would launch, so only the refusal side is checked on the CPU)
    st, _ = _lastrec(_dims(capacity=32, recent_window=0), n_valid=0, S=64, sink=0)
    assert st == _native.H2O_ERR_CAPACITY


def test_lastrec_rejects_bad_args():
    assert _lastrec(_dims(), 10, 8, sink=-1)[0] == _native.H2O_ERR_INVALID_ARG
    assert _lastrec(_dims(), 10, 8, sink=0, freed=None)[0] == _native.H2O_ERR_INVALID_ARG
    assert _lastrec(_dims(), 10, 0, sink=0)[0] == _native.H2O_ERR_INVALID_ARG
    assert _lastrec(_dims(head_dim=32), 10, 8, sink=0)[0] == _native.H2O_ERR_UNSUPPORTED


def test_chunk_attn_summed_weights_both_or_neither():
    d = _dims()
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, 0)
    for cs_cache, cs_new in ((FAKE, None), (None, FAKE)):
        st = h2o.lib.h2o_chunk_attn(ctypes.byref(d), ctypes.byref(cache), 0, 64, 0.125, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, cs_cache, cs_new, None, 0, None)
        assert st == _native.H2O_ERR_INVALID_ARG
        assert "colsum" in h2o.lib.h2o_last_error().decode()


def test_buffer_form_rejects_bad_args():
    d = _dims(capacity=256, recent_window=200)
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, 256)
    # selection: full cache, S + W > N_C
    st = h2o.lib.h2o_select_slots(ctypes.byref(d), ctypes.byref(cache), 1000, 64, 0, FAKE, None)
    assert st == _native.H2O_ERR_CAPACITY and cache.n_valid == 256
    assert h2o.lib.h2o_select_slots(ctypes.byref(_dims()), ctypes.byref(cache), 1000, 8, 9,
                                    FAKE, None) == _native.H2O_ERR_INVALID_ARG
    assert h2o.lib.h2o_select_slots(ctypes.byref(_dims()), ctypes.byref(cache), 1000, 8, 0,
                                    None, None) == _native.H2O_ERR_INVALID_ARG
    # attention over the buffer needs the targets and a workspace
    d = _dims()
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, 0)
    assert h2o.lib.h2o_buffer_attn(ctypes.byref(d), ctypes.byref(cache), 0, 64, 0.125, FAKE,
                                   FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                   None) == _native.H2O_ERR_INVALID_ARG
    st = h2o.lib.h2o_buffer_attn(ctypes.byref(d), ctypes.byref(cache), 0, 64, 0.125, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == _native.H2O_ERR_WORKSPACE
    # insertion needs its targets
    assert h2o.lib.h2o_insert(ctypes.byref(d), ctypes.byref(cache), 0, 64, FAKE, FAKE, None,
                              None, None) == _native.H2O_ERR_INVALID_ARG
    assert cache.n_valid == 0


def test_workspace_bytes_cover_both_attention_calls():
    d = _dims(capacity=8192, head_dim=128, n_q_heads=32, n_kv_heads=8)
    parts = 4 * 1 * 8 * (8192 + 1024) * 4
    words = 1 * 8 * (8192 // 64) * 8
    assert h2o.lib.h2o_workspace_bytes(ctypes.byref(d), 1024) == (parts + 255) // 256 * 256 + words
    f32 = _dims(dtype=_native.H2O_F32)
    assert h2o.lib.h2o_workspace_bytes(ctypes.byref(f32), 64) == 1 * 2 * 4 * 8


def test_workspace_bytes_invalid_is_zero():
    assert h2o.lib.h2o_workspace_bytes(None, 1) == 0
    assert h2o.lib.h2o_workspace_bytes(ctypes.byref(_dims(head_dim=3)), 1) == 0
    assert h2o.lib.h2o_workspace_bytes(ctypes.byref(_dims()), 0) == 0


def test_timer_rejects_bad_ids():
    assert h2o.lib.h2o_kernel_timer_start(99, 4) == _native.H2O_ERR_INVALID_ARG
    assert h2o.lib.h2o_kernel_timer_start(0, 0) == _native.H2O_ERR_INVALID_ARG
    ms, cnt = ctypes.c_double(), ctypes.c_int64()
    assert h2o.lib.h2o_kernel_timer_stop(-1, ctypes.byref(ms), ctypes.byref(cnt)) == \
        _native.H2O_ERR_INVALID_ARG


def test_python_binding_checks_shapes_before_calling():
    torch = pytest.importorskip("torch")
    d = h2o.H2ODims(1, 4, 2, 64, 256, 32, "bf16")
    q = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        h2o._need(q, (1, 4, 64, 64), torch.bfloat16, "q")     # CPU tensor refused
    with pytest.raises(ValueError):
        h2o._need(q.float(), (1, 4, 64, 64), torch.bfloat16, "q")
    assert d.group == 2


def test_noalloc_scratch_size():
    assert h2o.lib.h2o_noalloc_scratch_bytes() == 40 << 20


def _noalloc(dims, S, n_valid=0, cs=FAKE):
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, n_valid)
    return h2o.lib.h2o_chunk_attn_noalloc(ctypes.byref(dims), ctypes.byref(cache), 16384, S,
                                          0.125, FAKE, FAKE, FAKE, FAKE, FAKE, cs, cs, None)


def test_noalloc_rejects_workspace_beyond_scratch():
    """A decode step of 32 sequences x 8 KV heads x 4 query heads over 16384 slots needs
    67 MB of logits and partials, more than the 40 MiB scratch: refused before any GPU
    call (the pointers here are fake)."""
    dims = _dims(batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128, capacity=16384)
    need = h2o.lib.h2o_workspace_bytes(ctypes.byref(dims), 1)
    assert need > h2o.lib.h2o_noalloc_scratch_bytes()
    assert _noalloc(dims, 1, n_valid=16384) == _native.H2O_ERR_WORKSPACE
    assert "scratch" in h2o.lib.h2o_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=4, n_kv_heads=3), _native.H2O_ERR_INVALID_ARG),
    (dict(head_dim=96), _native.H2O_ERR_UNSUPPORTED),
])
def test_noalloc_validates_like_chunk_attn(kw, status):
    assert _noalloc(_dims(**kw), 64) == status


def _step(dims, n_valid=0, S=64, P=0, mode=_native.H2O_SCORE_H2O, cs=FAKE, freed=FAKE):
    cache = _native.CacheStruct(FAKE, FAKE, FAKE, FAKE, n_valid)
    return h2o.lib.h2o_chunk_step(ctypes.byref(dims), ctypes.byref(cache), P, S, 0.125, mode,
                                  FAKE, FAKE, FAKE, FAKE, FAKE, cs, cs, freed, None, 0, None)


@pytest.mark.parametrize("call,status", [
    (dict(mode=7), _native.H2O_ERR_INVALID_ARG),
    (dict(cs=None), _native.H2O_ERR_INVALID_ARG),
    (dict(freed=None), _native.H2O_ERR_INVALID_ARG),
    (dict(n_valid=257), _native.H2O_ERR_INVALID_ARG),
    # full cache, chunk 240 + window 32 > 256 slots: refused before the attention launches
    (dict(n_valid=256, S=240, P=1000), _native.H2O_ERR_CAPACITY),
])
def test_chunk_step_rejects_before_launch(call, status):
    assert _step(_dims(), **call) == status
    assert h2o.lib.h2o_last_error().decode()
