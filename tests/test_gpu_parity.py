"""HIP path vs the fp64 oracle, element by element, on seeded inputs (needs a GPU).

Every call goes through the C ABI (libh2o.so) via the ctypes binding.
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


def _chunk_getter(wl, layer=0):
    return lambda c: W.chunk_inputs(wl, layer, c)


def test_plumbing_f32_full_sequence():
    """Tiny plumbing workload (f32, d=64, GQA 2, N_C=256, W=32, S=64, 1024 tokens):
    all 16 chunks free-running, 4 filling and 12 evicting."""
    wl = W.WORKLOADS[1]
    swaps = H.run_chain(wl, range(wl.n_chunks), _chunk_getter(wl))
    print("near-tie swaps:", swaps)


@pytest.mark.parametrize("head_dim", [128, 64])
def test_bf16_chain_reduced(head_dim):
    """Qwen3-4B-like structure at reduced size (B=2, 8q/2kv heads, N_C=512, W=64,
    S=128, 2048 tokens): 4 filling and 12 evicting chunks, free-running."""
    wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=head_dim, capacity=512,
                    recent_window=64, chunk=128, seq_len=2048, heavy_count=20)
    swaps = H.run_chain(wl, range(wl.n_chunks), _chunk_getter(wl))
    print("near-tie swaps:", swaps)


def test_bf16_chain_h2o_norm():
    wl = W.workload(2, batch=1, n_q_heads=8, n_kv_heads=2, capacity=512, recent_window=64,
                    chunk=128, seq_len=1536, heavy_count=15)
    H.run_chain(wl, range(wl.n_chunks), _chunk_getter(wl), score_mode="h2o_norm")


def test_qwen3_shape_first_chunks():
    """Full Qwen3-4B attention shape, chunk 1k: the first two chunks (n = 0, 1024)."""
    wl = W.WORKLOADS[2]
    H.run_chain(wl, range(2), _chunk_getter(wl))


def _steady(wl, start, seed=0):
    s = W.steady_state(wl, 0, start=start, seed=seed)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    return cache, st


@pytest.mark.parametrize("key", [2, 3])
def test_steady_chunk_full_size(key):
    """One evicting chunk at the full configured size from a full cache
    (chunk 1k / N_C 8192 / W 256, and chunk 2k / N_C 16384 / W 512)."""
    wl = W.WORKLOADS[key]
    c = 16
    cache, st = _steady(wl, start=c * wl.chunk)
    H.run_chain(wl, [c], _chunk_getter(wl), cache=cache, st=st)


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", head_dim=64, n_q_heads=6, n_kv_heads=2, capacity=300, chunk=100,
         recent_window=10, seq_len=700),
    dict(dtype="bf16", head_dim=128, n_q_heads=3, n_kv_heads=3, capacity=97, chunk=33,
         recent_window=5, seq_len=330),
    dict(dtype="bf16", head_dim=128, n_q_heads=4, n_kv_heads=1, capacity=64, chunk=1,
         recent_window=3, seq_len=80),
    dict(dtype="f32", head_dim=128, n_q_heads=4, n_kv_heads=2, capacity=150, chunk=65,
         recent_window=7, seq_len=520),
    dict(dtype="f32", head_dim=64, n_q_heads=2, n_kv_heads=2, capacity=40, chunk=1,
         recent_window=2, seq_len=60),
    dict(dtype="bf16", head_dim=128, n_q_heads=6, n_kv_heads=2, capacity=70, chunk=1,
         recent_window=4, seq_len=90),
    dict(dtype="bf16", head_dim=128, n_q_heads=16, n_kv_heads=2, capacity=70, chunk=1,
         recent_window=4, seq_len=90),
], ids=["bf16_d64_g3_S100", "bf16_mha_S33", "bf16_S1", "f32_d128_S65", "f32_S1", "bf16_S1_g3",
        "bf16_S1_g8"])
def test_ragged_shapes(case):
    """Chunk lengths and capacities that are not tile multiples, MHA and GQA 3/4/8,
    single-token chunks (decode) at GQA 3, 4 and 8, and capacities that are not multiples
    of the chunk."""
    wl = W.workload(2, batch=2, heavy_count=4, sm_scale=case["head_dim"] ** -0.5, **case)
    H.run_chain(wl, range(wl.n_chunks), _chunk_getter(wl))


def _isolated_evict(wl, score_mode, seed):
    s = W.steady_state(wl, 0, start=20 * wl.chunk, seed=seed, tie_fraction=0.2)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    x = W.chunk_inputs(wl, 0, 20)
    cs_new = np.random.default_rng(seed).random((wl.batch, wl.n_kv_heads, wl.chunk)).astype(
        np.float32)
    k, v = H.dev(x["k"], torch.bfloat16), H.dev(x["v"], torch.bfloat16)
    freed = h2o.evict_and_insert(cache, st.P, k, v, H.dev(cs_new, torch.float32),
                                 score_mode=score_mode)
    torch.cuda.synchronize()
    victims = oracle.select_victims(st, wl.chunk, wl.recent_window, score_mode)
    want = oracle.evict_and_insert(st, victims, x["k"], x["v"], cs_new)
    return freed, cache, st, want


@pytest.mark.parametrize("score_mode", ["h2o", "h2o_norm"])
@pytest.mark.parametrize("seed", [0, 1])
def test_evict_isolated_bit_exact(score_mode, seed):
    """Same scores in, same victims out: selection and insertion are bit-exact at the
    full chunk-1k size, with 20% of the scores set to three shared values (ties)."""
    wl = W.WORKLOADS[2]
    freed, cache, st, want = _isolated_evict(wl, score_mode, seed)
    assert (H.host(freed) == want).all()
    assert (H.host(cache.pos) == st.pos).all()
    assert (H.host(cache.k) == st.K).all() and (H.host(cache.v) == st.V).all()
    assert (H.host(cache.score) == st.phi).all()
    assert cache.n_valid == st.n


@pytest.mark.parametrize("fill", ["all_equal", "two_levels"])
def test_evict_degenerate_scores(fill):
    """Every eligible score equal (the k-th key is the smallest key: the radix select runs
    no pass), or only two distinct values: victims are the lowest-index eligible slots."""
    wl = W.WORKLOADS[2]
    s = W.steady_state(wl, 0, start=20 * wl.chunk, seed=5, tie_fraction=0.0)
    phi = np.full_like(s["phi"], 3.0)
    if fill == "two_levels":
        phi[..., 1::3] = 2.0
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], phi, s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    x = W.chunk_inputs(wl, 0, 20)
    cs_new = np.ones((wl.batch, wl.n_kv_heads, wl.chunk), np.float32)
    k, v = H.dev(x["k"], torch.bfloat16), H.dev(x["v"], torch.bfloat16)
    freed = h2o.evict_and_insert(cache, st.P, k, v, H.dev(cs_new, torch.float32))
    torch.cuda.synchronize()
    victims = oracle.select_victims(st, wl.chunk, wl.recent_window)
    want = oracle.evict_and_insert(st, victims, x["k"], x["v"], cs_new)
    assert (H.host(freed) == want).all()
    assert (H.host(cache.pos) == st.pos).all()


def test_evict_isolated_large_capacity():
    wl = W.workload(3, capacity=32768, chunk=2048, recent_window=512)
    freed, cache, st, want = _isolated_evict(wl, "h2o", 3)
    assert (H.host(freed) == want).all()
    assert (H.host(cache.pos) == st.pos).all()


def test_update_scores_matches_oracle():
    wl = W.WORKLOADS[2]
    cache, st = _steady(wl, start=16 * wl.chunk)
    cs = np.random.default_rng(0).random((1, 8, wl.capacity)).astype(np.float32)
    h2o.update_scores(cache, H.dev(cs, torch.float32))
    oracle.update_scores(st, cs)
    torch.cuda.synchronize()
    got = H.host(cache.score)
    assert (H.rel_err(got, st.phi) <= 2 ** -23).all()     # one fp32 rounding


def test_determinism_bitwise():
    """Two runs of the same steady chunk give identical bits (no atomics in the reductions)."""
    wl = W.WORKLOADS[2]
    outs = []
    for _ in range(2):
        cache, st = _steady(wl, start=16 * wl.chunk)
        x = W.chunk_inputs(wl, 0, 16)
        g = H.gpu_chunk(cache, x, wl.sm_scale, wl.dtype)
        outs.append(g)
    for key in ("out", "lse", "colsum_cache", "colsum_new", "phi", "freed_slots"):
        assert (outs[0][key] == outs[1][key]).all(), key


def test_decode_steps_full_cache():
    """Decode workload (16 sequences, N_C 16384 full, W 512): the first 3 single-token
    steps, each with one eviction per (sequence, KV head)."""
    wl = W.WORKLOADS[5]
    s = W.decode_initial_state(wl)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    del s
    H.run_chain(wl, range(3), lambda t: W.decode_step_inputs(wl, t), cache=cache, st=st)


def test_layer_stack_first_chunks():
    """36-layer stack workload: the first two chunks (n = 0, 1024) of the last layer,
    whose inputs come from that layer's own seed."""
    wl = W.WORKLOADS[4]
    H.run_chain(wl, range(2), _chunk_getter(wl, layer=wl.layers - 1))


def test_layer_stack_interleaved_steady():
    """36-layer stack workload, chunk-major as a model runs it: layers 0, 17 and 35,
    each from its own full cache (its own seed), take chunks 64 and 65 in turn through
    one shared set of output and workspace buffers; each layer is compared with its
    own oracle state after every chunk."""
    wl = W.WORKLOADS[4]
    layers = (0, 17, wl.layers - 1)
    dt = H.TORCH_DT[wl.dtype]
    c0 = 64
    caches, states = {}, {}
    for layer in layers:
        s = W.steady_state(wl, layer, start=c0 * wl.chunk, seed=layer)
        states[layer] = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"],
                                                    s["n"], s["start"])
        caches[layer] = h2o.H2OCache(H.dims_of(wl), H.DEV)
        H.load_oracle_state(caches[layer], states[layer], wl.dtype)
    B, Hq, Hkv, D, NC, S = (wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity,
                            wl.chunk)
    bufs = {"out": torch.empty(B, Hq, S, D, dtype=dt, device=H.DEV),
            "lse": torch.empty(B, Hq, S, dtype=torch.float32, device=H.DEV),
            "colsum_cache": torch.empty(B, Hkv, NC, dtype=torch.float32, device=H.DEV),
            "colsum_new": torch.empty(B, Hkv, S, dtype=torch.float32, device=H.DEV),
            "freed_slots": torch.empty(B, Hkv, S, dtype=torch.int32, device=H.DEV),
            "workspace": torch.empty(max(1, h2o.workspace_bytes(H.dims_of(wl), S)),
                                     dtype=torch.uint8, device=H.DEV)}
    for c in (c0, c0 + 1):
        for layer in layers:
            cache, st = caches[layer], states[layer]
            where = f"layer {layer} chunk {c}:"
            x = W.chunk_inputs(wl, layer, c)
            n_before, pos_before, P = st.n, st.pos.copy(), st.P
            assert cache.next_pos == P == c * S
            got = h2o.step(cache, H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt),
                           wl.sm_scale, bufs=bufs)
            torch.cuda.synchronize()
            g = {key: H.host(t) for key, t in got.items()}
            r = oracle.h2o_step(st, x["q"], x["k"], x["v"], wl.sm_scale, wl.recent_window)
            H.compare_attention(g, r, n_before, wl.dtype, where)
            swaps = H.compare_victims(g["freed_slots"].astype(np.int64), r["freed_slots"],
                                      r["phi_updated"], pos_before, n_before, P,
                                      wl.recent_window, where)
            if swaps:
                H.load_oracle_state(cache, st, wl.dtype)
                continue
            assert (g["freed_slots"] == r["freed_slots"]).all(), f"{where} freed slots"
            assert (H.host(cache.pos) == st.pos).all(), f"{where} positions"
            assert torch.equal(cache.k, H.dev(st.K, dt)) and torch.equal(cache.v, H.dev(st.V, dt))
            e = H.rel_err(H.host(cache.score), st.phi).max()
            assert e <= H.TOL[wl.dtype]["cs_rel"], f"{where} scores rel {e:.3e}"


@pytest.mark.parametrize("score_mode", ["h2o", "h2o_norm"])
def test_decode_one_victim_fused_matches_separate(score_mode):
    """A decode step on a full cache takes one launch for selection and insertion; it
    gives bit for bit what the separate selection and insertion calls give, and the
    oracle's victim, with 20% of the scores set to three shared values (ties)."""
    wl = W.workload(5, batch=4)
    s = W.decode_initial_state(wl)
    phi = s["phi"].copy()
    r = np.random.default_rng(11)
    levels = np.sort(phi.reshape(-1))[[100, 1000, 4000]]
    mask = r.random(phi.shape) < 0.2
    phi[mask] = levels[r.integers(0, 3, mask.sum())]
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], phi, s["n"], s["start"])
    fused, sep = (h2o.H2OCache(H.dims_of(wl), H.DEV) for _ in range(2))
    for c in (fused, sep):
        H.load_oracle_state(c, st, wl.dtype)
    for t in range(3):
        x = W.decode_step_inputs(wl, t)
        P = fused.next_pos
        k, v = H.dev(x["k"], torch.bfloat16), H.dev(x["v"], torch.bfloat16)
        cs_new = H.dev(r.random((wl.batch, wl.n_kv_heads, 1)).astype(np.float32), torch.float32)
        f1 = h2o.evict_and_insert(fused, P, k, v, cs_new, score_mode=score_mode)
        f2 = h2o.select_slots(sep, P, 1, score_mode=score_mode)
        h2o.insert(sep, P, k, v, f2, cs_new)
        torch.cuda.synchronize()
        victims = oracle.select_victims(st, 1, wl.recent_window, score_mode)
        oracle.evict_and_insert(st, victims, x["k"], x["v"], H.host(cs_new))
        assert (H.host(f1) == victims).all(), f"step {t}: fused victim"
        assert torch.equal(f1, f2), f"step {t}: victims"
        for name in ("k", "v", "pos", "score"):
            assert torch.equal(getattr(fused, name), getattr(sep, name)), f"step {t}: {name}"
        assert (H.host(fused.pos) == st.pos).all()
        assert fused.n_valid == sep.n_valid == st.n


@pytest.mark.parametrize("score_mode", ["h2o", "h2o_norm"])
@pytest.mark.parametrize("case", ["steady_chunk", "decode", "filling", "f32_plumbing"])
def test_update_evict_fused_matches_separate(case, score_mode):
    """h2o_update_evict_and_insert gives bit for bit what h2o_update_scores followed by
    h2o_evict_and_insert gives: a full-size evicting chunk (k = 1024), a decode step (k = 1)
    and a filling chunk (k = 0, the update on its own)."""
    r = np.random.default_rng(21)
    if case == "decode":
        wl = W.workload(5, batch=4)
        s = W.decode_initial_state(wl)
        x = W.decode_step_inputs(wl, 0)
    elif case == "steady_chunk":
        wl = W.WORKLOADS[2]
        s = W.steady_state(wl, 0, start=20 * wl.chunk, seed=2, tie_fraction=0.2)
        x = W.chunk_inputs(wl, 0, 20)
    elif case == "f32_plumbing":
        wl = W.WORKLOADS[1]
        s = W.steady_state(wl, 0, start=10 * wl.chunk, seed=4, tie_fraction=0.2)
        x = W.chunk_inputs(wl, 0, 10)
    else:
        wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, capacity=512, recent_window=64,
                        chunk=128, seq_len=2048, heavy_count=20)
        st0 = oracle.H2OState.empty(wl.batch, wl.n_kv_heads, wl.capacity, wl.head_dim)
        for c in range(2):
            xc = W.chunk_inputs(wl, 0, c)
            oracle.h2o_step(st0, xc["q"], xc["k"], xc["v"], wl.sm_scale, wl.recent_window)
        s = {"k": st0.K, "v": st0.V, "pos": st0.pos, "phi": st0.phi, "n": st0.n, "start": st0.P}
        x = W.chunk_inputs(wl, 0, 2)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    fused, sep = (h2o.H2OCache(H.dims_of(wl), H.DEV) for _ in range(2))
    for c in (fused, sep):
        H.load_oracle_state(c, st, wl.dtype)
    S = x["k"].shape[2]
    dt = H.TORCH_DT[wl.dtype]
    k, v = H.dev(x["k"], dt), H.dev(x["v"], dt)
    cs_cache = H.dev(r.random((wl.batch, wl.n_kv_heads, wl.capacity)).astype(np.float32),
                     torch.float32)
    cs_new = H.dev(r.random((wl.batch, wl.n_kv_heads, S)).astype(np.float32), torch.float32)
    P = st.P
    f1 = h2o.update_evict_and_insert(fused, P, cs_cache, k, v, cs_new, score_mode=score_mode)
    h2o.update_scores(sep, cs_cache)
    f2 = h2o.evict_and_insert(sep, P, k, v, cs_new, score_mode=score_mode)
    torch.cuda.synchronize()
    assert torch.equal(f1, f2), "targets"
    for name in ("k", "v", "pos", "score"):
        assert torch.equal(getattr(fused, name), getattr(sep, name)), name
    assert fused.n_valid == sep.n_valid and fused.next_pos == sep.next_pos
    # and the oracle's targets on the updated scores (fp64 sums there: near ties at the
    # cut may swap, under the usual rule)
    oracle.update_scores(st, H.host(cs_cache))
    n_before, pos_before = st.n, st.pos.copy()
    rank = oracle.selection_scores(st.copy(), S, score_mode).copy()
    victims = oracle.select_victims(st, S, wl.recent_window, score_mode)
    want = oracle.evict_and_insert(st, victims, x["k"], x["v"], H.host(cs_new))
    H.compare_victims(H.host(f1).astype(np.int64), want, rank, pos_before, n_before, P,
                      wl.recent_window, case)
