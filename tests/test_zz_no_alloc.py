"""h2o_chunk_attn_noalloc against h2o_chunk_attn (needs a GPU).

The allocation-free entry point runs the same kernels with the library's static
device scratch as workspace, so its outputs must equal h2o_chunk_attn's bit for
bit.  Each test makes two calls in a row, the second with a smaller input, so the
second runs over the first one's leftovers in the shared scratch.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import gpu_harness as H  # noqa: E402
import h2o_sparse_attention_amd as h2o  # noqa: E402


def _both_ways(wl, st, x, summed_weights=True):
    """One chunk from oracle state st through both entry points; all outputs equal."""
    dt = H.TORCH_DT[wl.dtype]
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    P = st.P
    ref = h2o.chunk_attn(cache, P, q, k, v, wl.sm_scale, summed_weights=summed_weights)
    B, Hq, S, D = x["q"].shape
    Hkv, NC = wl.n_kv_heads, wl.capacity
    out = torch.full((B, Hq, S, D), float("nan"), dtype=dt, device=H.DEV)
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=H.DEV)
    cs_c = cs_n = None
    if summed_weights:
        cs_c = torch.full((B, Hkv, NC), float("nan"), dtype=torch.float32, device=H.DEV)
        cs_n = torch.full((B, Hkv, S), float("nan"), dtype=torch.float32, device=H.DEV)
    got = h2o.chunk_attn_noalloc(cache, P, q, k, v, wl.sm_scale, out, lse, cs_c, cs_n)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "lse", "colsum_cache", "colsum_new"), got, ref):
        if b is None:
            assert a is None
            continue
        assert torch.equal(a, b), f"{wl.name}: {name} differs from h2o_chunk_attn"


def _steady(wl, c, seed=0):
    s = W.steady_state(wl, 0, start=c * wl.chunk, seed=seed)
    return oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])


def test_noalloc_prefill_two_calls():
    """A full-size steady chunk (chunk 1k, 8192 slots: the split summed-weights partials
    live in the scratch), then a smaller chunk (B 2, 8q/2kv, 512 slots, chunk 128)."""
    wl = W.WORKLOADS[2]
    _both_ways(wl, _steady(wl, 16), W.chunk_inputs(wl, 0, 16))
    small = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, capacity=512, recent_window=64,
                       chunk=128, seq_len=4096, heavy_count=20)
    _both_ways(small, _steady(small, 20), W.chunk_inputs(small, 0, 20))


def test_noalloc_decode_two_calls():
    """Decode steps (split logits and partials in the scratch): 8 sequences over 16384
    slots, then 2 sequences over 4096 slots; and one step without summed weights."""
    wl = W.workload(5, batch=8)
    s = W.decode_initial_state(wl)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    _both_ways(wl, st, W.decode_step_inputs(wl, 0))
    small = W.workload(5, batch=2, capacity=4096)
    s = W.decode_initial_state(small)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    _both_ways(small, st, W.decode_step_inputs(small, 0))
    _both_ways(small, st, W.decode_step_inputs(small, 1), summed_weights=False)

