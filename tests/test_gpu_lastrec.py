"""lastrec policy and attention without summed weights: HIP path vs the fp64 oracle
(needs a GPU).  Every call goes through the C ABI via the ctypes binding.

lastrec ranks by position, so victims, freed slots, positions, cache rows and the
zero scores of inserted slots must match the oracle exactly; out and lse are held to
the attention tolerances of gpu_harness.
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


def _compare_out(g_out, g_lse, r, dtype, where):
    tol = H.TOL[dtype]
    H.check_out(g_out, r["out"], dtype, where)
    d_lse = np.abs(g_lse - r["lse"]).max()
    assert d_lse <= tol["lse_abs"], f"{where} lse abs {d_lse:.3e}"


def _compare_cache(cache, st, dtype, where):
    dt = H.TORCH_DT[dtype]
    assert cache.n_valid == st.n, where
    assert (H.host(cache.pos) == st.pos).all(), f"{where} pos"
    assert torch.equal(cache.k, H.dev(st.K, dt)) and torch.equal(cache.v, H.dev(st.V, dt)), \
        f"{where} cache rows"
    assert (H.host(cache.score) == st.phi).all(), f"{where} scores"


def run_lastrec_chain(wl, chunks, get_inputs, sink, cache=None, st=None):
    dims = H.dims_of(wl)
    cache = cache or h2o.H2OCache(dims, H.DEV)
    st = st or oracle.H2OState.empty(wl.batch, wl.n_kv_heads, wl.capacity, wl.head_dim)
    dt = H.TORCH_DT[wl.dtype]
    for c in chunks:
        x = get_inputs(c)
        assert cache.n_valid == st.n and cache.next_pos == st.P
        q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
        g = h2o.step(cache, q, k, v, wl.sm_scale, policy="lastrec", sink_tokens=sink)
        torch.cuda.synchronize()
        r = oracle.lastrec_step(st, x["q"], x["k"], x["v"], wl.sm_scale, sink)
        where = f"chunk {c}:"
        _compare_out(H.host(g["out"]), H.host(g["lse"]), r, wl.dtype, where)
        assert (H.host(g["freed_slots"]) == r["freed_slots"]).all(), f"{where} freed slots"
        _compare_cache(cache, st, wl.dtype, where)
    return cache, st


def test_lastrec_chain_bf16_reduced():
    """B=2, 8q/2kv heads, d=128, N_C=512, S=128, beta=32, 2048 tokens: 4 filling and
    12 evicting chunks; the cache ends holding the first 32 and the last 480 tokens."""
    wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, capacity=512, recent_window=64,
                    chunk=128, seq_len=2048, heavy_count=20)
    beta = 32
    cache, st = run_lastrec_chain(wl, range(wl.n_chunks), lambda c: W.chunk_inputs(wl, 0, c),
                                  beta)
    want = set(range(beta)) | set(range(2048 - (512 - beta), 2048))
    for b in range(2):
        for g in range(2):
            assert set(H.host(cache.pos)[b, g].tolist()) == want


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", head_dim=64, n_q_heads=6, n_kv_heads=2, capacity=300, chunk=100,
         seq_len=700, sink=7),
    dict(dtype="bf16", head_dim=128, n_q_heads=4, n_kv_heads=1, capacity=64, chunk=1,
         seq_len=80, sink=4),
    dict(dtype="f32", head_dim=128, n_q_heads=4, n_kv_heads=2, capacity=150, chunk=65,
         seq_len=520, sink=20),
    dict(dtype="f32", head_dim=64, n_q_heads=2, n_kv_heads=2, capacity=40, chunk=1,
         seq_len=60, sink=0),
], ids=["bf16_d64_g3_S100", "bf16_S1_decode", "f32_d128_S65", "f32_S1_nosink"])
def test_lastrec_ragged(case):
    """Ragged chunk lengths and capacities, single-token chunks (the bf16 one takes the
    split decode kernels without summed weights), beta = 0."""
    case = dict(case)
    sink = case.pop("sink")
    wl = W.workload(2, batch=2, heavy_count=4, recent_window=0,
                    sm_scale=case["head_dim"] ** -0.5, **case)
    run_lastrec_chain(wl, range(wl.n_chunks), lambda c: W.chunk_inputs(wl, 0, c), sink)


def test_lastrec_one_victim_with_empty_targets():
    """N_C = 11, S = 3, beta = 2: the fourth chunk's targets are one victim (the oldest
    non-sink token) and the two empty slots; later chunks evict 3 each."""
    wl = W.workload(2, batch=2, n_q_heads=4, n_kv_heads=2, capacity=11, recent_window=0,
                    chunk=3, seq_len=30, heavy_count=3)
    cache, st = run_lastrec_chain(wl, range(wl.n_chunks), lambda c: W.chunk_inputs(wl, 0, c), 2)
    want = {0, 1} | set(range(30 - 9, 30))
    for b in range(2):
        for g in range(2):
            assert set(H.host(cache.pos)[b, g].tolist()) == want


@pytest.mark.parametrize("key,sink", [(2, 64), (3, 1000), ("max", 4)])
def test_lastrec_isolated_full_size(key, sink):
    """Eviction alone from a full cache in random slot order (chunk 1k / N_C 8192,
    chunk 2k / N_C 16384, and chunk 1k at the 32768-slot maximum with 8 query / 2 KV
    heads): same victims, rows, positions and zero scores as the oracle."""
    if key == "max":
        wl = W.workload(2, batch=1, n_q_heads=8, n_kv_heads=2, capacity=32768,
                        recent_window=512, chunk=1024, seq_len=65536)
        c, seed = 40, 4
    else:
        wl, c, seed = W.WORKLOADS[key], 20, key
    s = W.steady_state(wl, 0, start=c * wl.chunk, seed=seed)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    x = W.chunk_inputs(wl, 0, c)
    k, v = H.dev(x["k"], torch.bfloat16), H.dev(x["v"], torch.bfloat16)
    freed = h2o.evict_and_insert_lastrec(cache, st.P, k, v, sink)
    torch.cuda.synchronize()
    victims = oracle.select_victims_lastrec(st, wl.chunk, sink)
    want = oracle.evict_and_insert(st, victims, x["k"], x["v"],
                                   np.zeros((wl.batch, wl.n_kv_heads, wl.chunk)))
    assert (H.host(freed) == want).all()
    _compare_cache(cache, st, wl.dtype, "isolated")


def test_lastrec_decode_full_cache():
    """Decode workload (16 sequences, N_C 16384 full), beta = 4: three single-token steps,
    each evicting the oldest non-sink slot of every (sequence, KV head)."""
    wl = W.WORKLOADS[5]
    s = W.decode_initial_state(wl)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    del s
    run_lastrec_chain(wl, range(3), lambda t: W.decode_step_inputs(wl, t), 4, cache=cache,
                      st=st)
    assert (H.host(cache.pos)[:, :, 4:7] == np.arange(16384, 16387)).all()


def test_lastrec_decode_max_capacity():
    """Decode at the 32768-slot maximum (two sequences, 8 query / 2 KV heads), beta = 4:
    three single-token steps over eight 4096-slot splits, each evicting the oldest
    non-sink slot."""
    wl = W.workload(5, batch=2, n_q_heads=8, n_kv_heads=2, capacity=32768)
    s = W.decode_initial_state(wl)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    del s
    run_lastrec_chain(wl, range(3), lambda t: W.decode_step_inputs(wl, t), 4, cache=cache,
                      st=st)
    assert (H.host(cache.pos)[:, :, 4:7] == np.arange(32768, 32771)).all()


def _attn_both_ways(wl, cache, x):
    dt = H.TORCH_DT[wl.dtype]
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    P = cache.next_pos
    with_cs = h2o.chunk_attn(cache, P, q, k, v, wl.sm_scale)
    without = h2o.chunk_attn(cache, P, q, k, v, wl.sm_scale, summed_weights=False)
    torch.cuda.synchronize()
    assert without[2] is None and without[3] is None
    assert torch.equal(with_cs[0], without[0]), "out differs without summed weights"
    assert torch.equal(with_cs[1], without[1]), "lse differs without summed weights"


def test_attention_without_summed_weights_is_identical():
    """Skipping the summed weights changes nothing else: out and lse are bit-identical
    for a steady chunk-1k step and for a decode step."""
    wl = W.WORKLOADS[2]
    s = W.steady_state(wl, 0, start=16 * wl.chunk)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    _attn_both_ways(wl, cache, W.chunk_inputs(wl, 0, 16))

    wl = W.WORKLOADS[5]
    s = W.decode_initial_state(wl, batches=range(2))
    wl = W.workload(5, batch=2)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    x = W.decode_step_inputs(W.WORKLOADS[5], 0)
    x = {key: val[:2] if isinstance(val, np.ndarray) else val for key, val in x.items()}
    _attn_both_ways(wl, cache, x)
