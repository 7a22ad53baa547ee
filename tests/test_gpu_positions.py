"""The implicit positional mask on the GPU (needs a GPU).

"Kernel Support Needs" (montaan paper page) states the causal mask through the
slot positions: key j is visible to query row i iff t(j) <= P + i (an empty
slot, t = -1, never).  A cache built by this library's own insertions only
holds earlier tokens, 0 <= t(j) < P; these tests load caches that break that
(filled slots marked -1, slots holding tokens at or after the chunk start) and
check the HIP path against the hand-derived worked examples of
tests/golden/h2o_worked_examples.json and against the fp64 oracle.
"""
import json

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
from oracle_pins import GOLDEN, _vals  # noqa: E402

with open(GOLDEN) as _f:
    CASES = json.load(_f)["cases"]


def _bf16_exact(xs):
    x = np.asarray(xs, np.float64).astype(np.float32)
    return (W.bf16_round(x).astype(np.float64) == np.asarray(xs, np.float64)).all()


def _golden_params():
    out = []
    for case in CASES:
        for dtype in ("f32", "bf16"):
            st, ch = case["state"], case["chunk"]
            exact = all(_bf16_exact(np.ravel(v)) for v in (st["k"], st["v"], ch["q"], ch["k"],
                                                            ch["v"]))
            if dtype == "bf16" and not exact:
                continue              # the hand-derived values hold for the exact inputs only
            for d in (64, 128):
                out.append(pytest.param(case["name"], dtype, d,
                                        id=f"{case['name']}-{dtype}-d{d}"))
    return out


@pytest.mark.parametrize("name,dtype,head_dim", _golden_params())
def test_golden_worked_examples(name, dtype, head_dim):
    """Each worked example with its one-dimensional vectors placed in coordinate 0 of
    head_dim-wide rows: outputs, log-sum-exp, summed weights, targets, positions and
    scores against the hand-derived values."""
    case = next(c for c in CASES if c["name"] == name)
    dims_j, st, ch, ex = case["dims"], case["state"], case["chunk"], case["expect"]
    NC, Hq, S = dims_j["capacity"], dims_j["Hq"], len(ch["k"])
    dims = h2o.H2ODims(1, Hq, 1, head_dim, NC, dims_j["W"], dtype)
    dt = H.TORCH_DT[dtype]

    def rows(vals, shape):
        a = np.zeros(shape + (head_dim,))
        a[..., 0] = np.asarray(vals, np.float64).reshape(shape)
        return H.dev(a, dt)

    cache = h2o.H2OCache(dims, H.DEV)
    cache.load(rows(st["k"], (1, 1, NC)), rows(st["v"], (1, 1, NC)),
               H.dev(np.array(st["pos"], np.int32).reshape(1, 1, NC), torch.int32),
               H.dev(_vals(st["phi"]).reshape(1, 1, NC).astype(np.float32), torch.float32),
               st["n"], st["P"])
    q = rows(ch["q"], (1, Hq, S))
    k, v = rows(ch["k"], (1, 1, S)), rows(ch["v"], (1, 1, S))
    P = st["P"]
    out, lse, cs_cache, cs_new = h2o.chunk_attn(cache, P, q, k, v, dims_j["sm_scale"])
    h2o.update_scores(cache, cs_cache)
    phi_upd = cache.score.clone()
    freed = h2o.evict_and_insert(cache, P, k, v, cs_new,
                                 score_mode=dims_j.get("score_mode", "h2o"))
    torch.cuda.synchronize()

    tol = H.TOL[dtype]
    want_out = np.zeros((1, Hq, S, head_dim))
    want_out[..., 0] = _vals(ex["out"]).reshape(1, Hq, S)
    H.check_out(H.host(out), want_out, dtype, name)
    assert np.abs(H.host(lse).reshape(-1) - _vals(ex["lse"])).max() <= tol["lse_abs"]

    def close(got, want, what):
        got = np.asarray(got, np.float64).reshape(-1)
        want = np.asarray(want, np.float64).reshape(-1)
        zero = want == 0
        assert (got[zero] == 0).all(), f"{name}: {what} not zero where expected"
        e = H.rel_err(got[~zero], want[~zero]).max(initial=0.0)
        assert e <= tol["cs_rel"], f"{name}: {what} rel {e:.3e}"

    close(H.host(cs_cache), _vals(ex["colsum_cache"]), "colsum_cache")
    close(H.host(cs_new), _vals(ex["colsum_new"]), "colsum_new")
    close(H.host(phi_upd)[..., :st["n"]], _vals(ex["phi_updated"])[:st["n"]], "phi_updated")
    assert H.host(freed).reshape(-1).tolist() == ex["freed_slots"]
    assert H.host(cache.pos).reshape(-1).tolist() == ex["pos_after"]
    close(H.host(cache.score), _vals(ex["phi_after"]), "phi_after")
    assert cache.n_valid == ex["n_after"] and cache.next_pos == ex["P_after"]


def _scramble_positions(st, S, seed, frac=0.04):
    """Mark a fraction of the filled slots empty (-1) and give another fraction
    positions at or after the chunk start (some past the chunk's last row)."""
    r = np.random.default_rng(seed)
    B, Hkv, _ = st.pos.shape
    for b in range(B):
        for g in range(Hkv):
            idx = r.choice(st.n, 2 * max(1, int(frac * st.n)), replace=False)
            half = idx.size // 2
            st.pos[b, g, idx[:half]] = -1
            st.pos[b, g, idx[half:]] = st.P + r.integers(0, S + 64, idx.size - half)


@pytest.mark.parametrize("shape", ["reduced_d128", "reduced_d64", "reduced_f32", "headline"])
def test_cache_positions_outside_chunk_start(shape):
    """A cache whose filled slots include empty-marked slots and slots holding tokens
    at or after the chunk start: one chunk (attention, summed weights, update,
    eviction, insertion) against the oracle's literal positional mask."""
    if shape == "headline":
        wl = W.WORKLOADS[2]
        c = 16
    else:
        d = 64 if shape == "reduced_d64" else 128
        dtype = "f32" if shape == "reduced_f32" else "bf16"
        wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=d, capacity=500,
                        recent_window=64, chunk=128, seq_len=4096, heavy_count=20,
                        dtype=dtype, sm_scale=d ** -0.5)
        c = 20
    s = W.steady_state(wl, 0, start=c * wl.chunk, seed=3)
    n = wl.capacity - (37 if shape != "headline" else 0)      # a partial last tile
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], n, s["start"])
    st.pos[:, :, n:] = -1
    _scramble_positions(st, wl.chunk, seed=5)
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    H.run_chain(wl, [c], lambda cc: W.chunk_inputs(wl, 0, cc), cache=cache, st=st)


def test_decode_positions_outside_step():
    """Single-token steps (the split decode kernels) over a full cache with empty-marked
    slots and slots holding later positions."""
    wl = W.workload(5, batch=2)
    s = W.decode_initial_state(wl)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    _scramble_positions(st, 1, seed=6, frac=0.01)
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    H.run_chain(wl, range(2), lambda t: W.decode_step_inputs(wl, t), cache=cache, st=st)
