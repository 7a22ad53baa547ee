"""HIP graph capture of the library's calls (needs a GPU).

A caller may capture a chunk step, a decode step or a backward into a HIP graph
and replay it (bench.py times its lines that way).  Each test runs the call
eagerly, captures it once, then replays the graph several times.  Before each
replay the mutable state (the cache) is restored, and some unrelated eager work
and a synchronisation run between replays.  Every replay must give the eager
results bit for bit: the kernels are deterministic, so any difference means a
captured launch read or wrote something other than on the eager run.
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

REPLAYS = 3


class Snapshot:
    """The cache's device tensors and host counters, restorable in place."""

    def __init__(self, cache: h2o.H2OCache):
        self.cache = cache
        self.t = [x.clone() for x in (cache.k, cache.v, cache.pos, cache.score)]
        self.n, self.p = cache.n_valid, cache.next_pos

    def restore(self):
        for dst, src in zip((self.cache.k, self.cache.v, self.cache.pos, self.cache.score), self.t):
            dst.copy_(src)
        self.cache.n_valid, self.cache.next_pos = self.n, self.p


def _capture(fn, restore):
    """One warm run on a side stream (as torch requires), then the capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        restore()
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        res = fn()
    torch.cuda.synchronize()
    return graph, res


def _unrelated_work():
    a = torch.randn(512, 512, device=H.DEV)
    (a @ a).sum().item()


def _check_replays(fn, snap, outputs):
    """Eager run, capture, REPLAYS replays; outputs(res) lists the tensors compared."""
    snap.restore()
    want = [t.clone() for t in outputs(fn())]
    torch.cuda.synchronize()
    graph, res = _capture(fn, snap.restore)
    for r in range(REPLAYS):
        snap.restore()
        _unrelated_work()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (g, w) in enumerate(zip(outputs(res), want)):
            assert torch.equal(g, w), f"replay {r}: output {i} differs from the eager run"


def _steady_cache(wl, chunk_index):
    s = W.steady_state(wl, 0, start=chunk_index * wl.chunk)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    return cache, st


@pytest.mark.parametrize("policy", ["h2o", "lastrec", "h2o_buffer"])
def test_step_graph_replays(policy):
    """One evicting chunk (B=2, 8q/2kv heads, N_C=512, S=128) per policy, as h2o.step
    issues it: the whole chunk step, the lastrec pair of calls, or the buffer form's
    four calls."""
    wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, capacity=512, recent_window=64,
                    chunk=128, seq_len=2048, heavy_count=20)
    cache, st = _steady_cache(wl, 6)
    x = W.chunk_inputs(wl, 0, 6)
    dt = H.TORCH_DT[wl.dtype]
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    snap = Snapshot(cache)
    kw = dict(policy=policy, sink_tokens=4 if policy == "lastrec" else 0)

    def fn():
        return h2o.step(cache, q, k, v, wl.sm_scale, **kw)

    def outputs(res):
        return [res[n] for n in sorted(res)] + [cache.k, cache.v, cache.pos, cache.score]

    _check_replays(fn, snap, outputs)


def test_chunk_step_graph_replays_full_size():
    """The steady full-cache chunk of the chunk-1k / 64k-context workload (1024 queries,
    8192 slots, 32q/8kv heads) through h2o_chunk_step."""
    wl = W.WORKLOADS[2]
    cache, st = _steady_cache(wl, 16)
    x = W.chunk_inputs(wl, 0, 16)
    dt = H.TORCH_DT[wl.dtype]
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    snap = Snapshot(cache)

    def fn():
        return h2o.chunk_step(cache, st.P, q, k, v, wl.sm_scale)

    def outputs(res):
        return list(res) + [cache.k, cache.v, cache.pos, cache.score]

    _check_replays(fn, snap, outputs)


@pytest.mark.parametrize("score_mode", ["h2o", "h2o_norm"])
def test_decode_step_graph_replays(score_mode):
    """A full-cache decode step (4 sequences, 32q/8kv heads, N_C 16384): the splits
    exchange their (m, l) inside the attention launch, with flags cleared by a kernel
    of the same call."""
    wl = W.workload(5, batch=4)
    s = W.decode_initial_state(wl)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    x = W.decode_step_inputs(wl, 0)
    dt = H.TORCH_DT[wl.dtype]
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    snap = Snapshot(cache)

    def fn():
        return h2o.chunk_step(cache, st.P, q, k, v, wl.sm_scale, score_mode)

    def outputs(res):
        return list(res) + [cache.k, cache.v, cache.pos, cache.score]

    _check_replays(fn, snap, outputs)


def test_backward_graph_replays_full_size():
    """The backward of a steady full-size chunk: the dQ kernel runs on the library's
    second stream, forked from and joined back to the capturing stream."""
    wl = W.WORKLOADS[2]
    cache, st = _steady_cache(wl, 16)
    x = W.chunk_inputs(wl, 0, 16)
    dt = H.TORCH_DT[wl.dtype]
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    out, lse, _, _ = h2o.chunk_attn(cache, st.P, q, k, v, wl.sm_scale, summed_weights=False)
    r = np.random.default_rng(5)
    dout = H.dev(W.synth.bf16_round(r.standard_normal(tuple(out.shape)).astype(np.float32)), dt)
    snap = Snapshot(cache)

    def fn():
        return h2o.chunk_attn_backward(cache, st.P, q, k, v, out, lse, dout, wl.sm_scale)

    _check_replays(fn, snap, list)
