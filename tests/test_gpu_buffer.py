"""Insert-first buffer form: HIP path vs the fp64 oracle (needs a GPU).

The oracle follows the pages' order literally (victims on the scores before the
chunk, the chunk written into the buffer, attention over the N_C slots under the
positional mask, scores accumulated); the HIP path selects the targets, attends
with the overwritten slots excluded and the chunk's keys causal, updates the
scores and inserts.  Every call goes through the C ABI via the ctypes binding.

Victim sets must match the oracle's exactly, except that swaps across the cut
between scores within 1e-5 (relative) are accepted; the chunk then goes on with
the oracle's targets, so its attention is still compared on the same keys.
Attention and summed-weight tolerances are those of gpu_harness.
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


def buffer_chunk(cache, st, x, wl, score_mode="h2o", where=""):
    dt = H.TORCH_DT[wl.dtype]
    tol = H.TOL[wl.dtype]
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    P, S = cache.next_pos, x["q"].shape[2]
    assert cache.n_valid == st.n and P == st.P
    n_before, pos_before = st.n, st.pos.copy()
    rank = oracle.selection_scores(st.copy(), S, score_mode).copy()
    freed = h2o.select_slots(cache, P, S, score_mode=score_mode)
    torch.cuda.synchronize()
    r = oracle.buffer_step(st, x["q"], x["k"], x["v"], wl.sm_scale, wl.recent_window,
                           score_mode)
    g_freed = H.host(freed).astype(np.int64)
    swaps = H.compare_victims(g_freed, r["freed_slots"], rank, pos_before, n_before, P,
                              wl.recent_window, where)
    if swaps:
        freed = H.dev(r["freed_slots"].astype(np.int32), torch.int32)
    else:
        assert (g_freed == r["freed_slots"]).all(), f"{where} targets"
    out, lse, cs_cache, cs_new = h2o.buffer_attn(cache, P, q, k, v, freed, wl.sm_scale)
    h2o.update_scores(cache, cs_cache)
    h2o.insert(cache, P, k, v, freed, cs_new)
    torch.cuda.synchronize()

    # attention
    g = {"out": H.host(out), "lse": H.host(lse)}
    H.check_out(g["out"], r["out"], wl.dtype, where)
    assert np.abs(g["lse"] - r["lse"]).max() <= tol["lse_abs"], f"{where} lse"
    # summed weights: survivors keep their slot; chunk token i' is the slot it went to
    csc, csn = H.host(cs_cache), H.host(cs_new)
    fr = H.host(freed).astype(np.int64)
    B, Hkv = fr.shape[:2]
    for b in range(B):
        for gh in range(Hkv):
            victims = fr[b, gh][fr[b, gh] < n_before]
            surv = np.setdiff1d(np.arange(n_before), victims)
            e1 = H.rel_err(csc[b, gh, surv], r["colsum"][b, gh, surv]).max(initial=0.0)
            assert e1 <= tol["cs_rel"], f"{where} survivors' summed weights rel {e1:.3e}"
            assert (csc[b, gh, victims] == 0).all(), f"{where} overwritten slots not zero"
            assert (csc[b, gh, n_before:] == 0).all(), f"{where} empty slots not zero"
            e2 = H.rel_err(csn[b, gh], r["colsum"][b, gh, fr[b, gh]]).max()
            assert e2 <= tol["cs_rel"], f"{where} chunk keys' summed weights rel {e2:.3e}"
    # the cache after the chunk
    assert cache.n_valid == st.n
    assert (H.host(cache.pos) == st.pos).all(), f"{where} positions"
    assert torch.equal(cache.k, H.dev(st.K, dt)) and torch.equal(cache.v, H.dev(st.V, dt)), \
        f"{where} cache rows"
    e = H.rel_err(H.host(cache.score)[:, :, :st.n], st.phi[:, :, :st.n]).max()
    assert e <= tol["cs_rel"], f"{where} scores rel {e:.3e}"
    if swaps:
        H.load_oracle_state(cache, st, wl.dtype)
    return swaps


def run_buffer_chain(wl, chunks, get_inputs, score_mode="h2o", cache=None, st=None):
    cache = cache or h2o.H2OCache(H.dims_of(wl), H.DEV)
    st = st or oracle.H2OState.empty(wl.batch, wl.n_kv_heads, wl.capacity, wl.head_dim)
    swaps = 0
    for c in chunks:
        swaps += buffer_chunk(cache, st, get_inputs(c), wl, score_mode, where=f"chunk {c}:")
    return swaps


def _chunks(wl):
    return lambda c: W.chunk_inputs(wl, 0, c)


def test_buffer_plumbing_f32_full_sequence():
    """Plumbing workload (f32, N_C 256, S 64, 1024 tokens): 4 filling, 12 evicting chunks."""
    wl = W.WORKLOADS[1]
    print("near-tie swaps:", run_buffer_chain(wl, range(wl.n_chunks), _chunks(wl)))


@pytest.mark.parametrize("head_dim", [128, 64])
def test_buffer_chain_bf16_reduced(head_dim):
    """B=2, 8q/2kv heads, N_C=512, W=64, S=128, 2048 tokens, free-running."""
    wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=head_dim, capacity=512,
                    recent_window=64, chunk=128, seq_len=2048, heavy_count=20)
    print("near-tie swaps:", run_buffer_chain(wl, range(wl.n_chunks), _chunks(wl)))


def test_buffer_chain_h2o_norm():
    wl = W.workload(2, batch=1, n_q_heads=8, n_kv_heads=2, capacity=512, recent_window=64,
                    chunk=128, seq_len=1536, heavy_count=15)
    run_buffer_chain(wl, range(wl.n_chunks), _chunks(wl), score_mode="h2o_norm")


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", head_dim=64, n_q_heads=6, n_kv_heads=2, capacity=300, chunk=100,
         recent_window=10, seq_len=700),
    dict(dtype="bf16", head_dim=128, n_q_heads=4, n_kv_heads=1, capacity=64, chunk=1,
         recent_window=3, seq_len=80),
    dict(dtype="f32", head_dim=128, n_q_heads=4, n_kv_heads=2, capacity=150, chunk=65,
         recent_window=7, seq_len=520),
    dict(dtype="f32", head_dim=64, n_q_heads=2, n_kv_heads=2, capacity=40, chunk=1,
         recent_window=2, seq_len=60),
], ids=["bf16_d64_g3_S100", "bf16_S1_decode", "f32_d128_S65", "f32_S1"])
def test_buffer_ragged(case):
    """Ragged chunk lengths and capacities; single-token chunks (the bf16 one takes the
    split decode kernels with the overwritten slot excluded)."""
    wl = W.workload(2, batch=2, heavy_count=4, sm_scale=case["head_dim"] ** -0.5, **case)
    run_buffer_chain(wl, range(wl.n_chunks), _chunks(wl))


@pytest.mark.parametrize("score_mode", ["h2o", "h2o_norm"])
def test_buffer_one_victim_with_empty_targets(score_mode):
    """N_C = 11, S = 3, W = 5: the fourth chunk's targets are one victim and the two
    empty slots (k = 1 with S > 1), later chunks evict 3 each."""
    wl = W.workload(2, batch=2, n_q_heads=4, n_kv_heads=2, capacity=11, recent_window=5,
                    chunk=3, seq_len=30, heavy_count=3)
    run_buffer_chain(wl, range(wl.n_chunks), _chunks(wl), score_mode=score_mode)


def test_buffer_select_one_victim_full_size():
    """h2o_select_slots on an 8192-slot cache holding 7169 tokens, chunk 1024: the
    targets are the one oracle victim and the 1023 empty slots."""
    wl = W.WORKLOADS[2]
    s = W.steady_state(wl, 0, start=20 * wl.chunk, seed=9, tie_fraction=0.2)
    n = wl.capacity - wl.chunk + 1
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], n, s["start"])
    st.pos[:, :, n:] = -1
    st.phi[:, :, n:] = 0.0
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    freed = h2o.select_slots(cache, st.P, wl.chunk)
    torch.cuda.synchronize()
    victims = oracle.select_victims(st, wl.chunk, wl.recent_window)
    want = np.concatenate([victims, np.broadcast_to(np.arange(n, wl.capacity),
                                                    victims.shape[:2] + (wl.chunk - 1,))],
                          axis=2)
    assert (H.host(freed) == want).all()


@pytest.mark.parametrize("key", [2, 3])
def test_buffer_steady_chunk_full_size(key):
    """One chunk at the full configured size from a full cache in random slot order
    (chunk 1k / N_C 8192, chunk 2k / N_C 16384): 1024 / 2048 slots excluded."""
    wl = W.WORKLOADS[key]
    c = 16
    s = W.steady_state(wl, 0, start=c * wl.chunk)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    run_buffer_chain(wl, [c], _chunks(wl), cache=cache, st=st)


def test_buffer_decode_full_cache():
    """Decode workload (16 sequences, N_C 16384 full, W 512): three single-token steps,
    each attending without the slot it is about to overwrite."""
    wl = W.WORKLOADS[5]
    s = W.decode_initial_state(wl)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    del s
    run_buffer_chain(wl, range(3), lambda t: W.decode_step_inputs(wl, t), cache=cache, st=st)


def test_buffer_steady_chunk_max_capacity():
    """The buffer form at the largest capacity (32768 slots, chunk 1k, 8 query / 2 KV
    heads): 1024 of 32768 slots excluded, the exclusion bits at their 512-word limit."""
    wl = W.workload(2, batch=1, n_q_heads=8, n_kv_heads=2, capacity=32768, recent_window=512,
                    chunk=1024, seq_len=65536)
    c = 40
    s = W.steady_state(wl, 0, start=c * wl.chunk)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    run_buffer_chain(wl, [c], _chunks(wl), cache=cache, st=st)
