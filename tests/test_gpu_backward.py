"""Backward of the chunk attention: HIP path vs the fp64 oracle (needs a GPU).

The GPU backward receives the GPU forward's own out and lse (as a training step
would); the oracle recomputes everything in fp64 from the same input bits.

Tolerances.  f32: max |err| <= 1e-4 * max|ref| per gradient tensor, relative
L2 <= 1e-5.  bf16: the weights m and the ds values are rounded to bf16 (2^-9
relative each) for their MFMA products, and D_i uses the bf16-stored output,
so each product carries up to about 2^-8 relative error; ds sums to zero along
each row, so a per-element relative bound is meaningless for dQ.  The bound is
per tensor: max |err| <= 1e-2 * max|ref| and relative L2 <= 5e-3 (1.3 x 2^-8;
the errors of independent terms partly cancel, about 1.7e-3 is typical).

The workspace is filled with NaN bytes first, so a value the kernels read from
it without having written it shows up as NaN in the gradients.
"""
import ctypes

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

TOL = {"f32": dict(max_rel=1e-4, l2=1e-5), "bf16": dict(max_rel=1e-2, l2=5e-3)}
NAMES = ("dq", "dk_new", "dv_new", "dk_cache", "dv_cache")


def _dout(wl, S, seed):
    r = np.random.default_rng(1000 + seed)
    x = r.standard_normal((wl.batch, wl.n_q_heads, S, wl.head_dim)).astype(np.float32)
    return W.synth.bf16_round(x) if wl.dtype == "bf16" else x


def _workspace(wl, S):
    d = H.dims_of(wl).c()
    ws = torch.empty(int(h2o.lib.h2o_backward_workspace_bytes(ctypes.byref(d), S)),
                     dtype=torch.uint8, device=H.DEV)
    ws.fill_(255)
    return ws


def check_backward(wl, st, x, seed=0, freed=None, where=""):
    """Forward on the GPU from oracle state ``st``, then the backward, against the oracle."""
    dt = H.TORCH_DT[wl.dtype]
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    S = x["q"].shape[2]
    P = st.P
    fr = None if freed is None else H.dev(freed.astype(np.int32), torch.int32)
    if fr is None:
        out, lse, _, _ = h2o.chunk_attn(cache, P, q, k, v, wl.sm_scale, summed_weights=False)
    else:
        out, lse, _, _ = h2o.buffer_attn(cache, P, q, k, v, fr, wl.sm_scale, summed_weights=False)
    dout_np = _dout(wl, S, seed)
    got = h2o.chunk_attn_backward(cache, P, q, k, v, out, lse, H.dev(dout_np, dt), wl.sm_scale,
                                  freed_slots=fr, workspace=_workspace(wl, S))
    torch.cuda.synchronize()
    excl = None
    if freed is not None:
        excl = np.zeros((wl.batch, wl.n_kv_heads, wl.capacity), bool)
        for b in range(wl.batch):
            for g in range(wl.n_kv_heads):
                vs = freed[b, g][freed[b, g] < st.n]
                excl[b, g, vs] = True
    want = oracle.attend_chunk_backward(st, x["q"], x["k"], x["v"], dout_np, wl.sm_scale,
                                        excluded=excl)
    tol = TOL[wl.dtype]
    for name, gt, wt in zip(NAMES, got, want):
        gv = H.host(gt)
        scale = np.abs(wt).max()
        err = np.abs(gv - wt).max()
        l2 = np.linalg.norm(gv - wt) / max(np.linalg.norm(wt), 1e-30)
        print(f"{where} {name}: max|ref| {scale:.3e} max err {err:.3e} rel-L2 {l2:.2e}")
        assert err <= tol["max_rel"] * scale, f"{where} {name} max err {err:.3e} vs {scale:.3e}"
        assert l2 <= tol["l2"], f"{where} {name} rel-L2 {l2:.3e}"
    # slots past n_valid and excluded slots have zero gradient
    for gt in got[3:]:
        gv = H.host(gt)
        assert (gv[:, :, st.n:] == 0).all()
        if excl is not None:
            assert (gv[excl] == 0).all()


def _state_after(wl, chunks):
    """Oracle state after the first `chunks` chunks of the workload (attend-first h2o)."""
    st = oracle.H2OState.empty(wl.batch, wl.n_kv_heads, wl.capacity, wl.head_dim)
    for c in range(chunks):
        x = W.chunk_inputs(wl, 0, c)
        oracle.h2o_step(st, x["q"], x["k"], x["v"], wl.sm_scale, wl.recent_window)
    return st


@pytest.mark.parametrize("chunk", [0, 6])
def test_backward_f32_plumbing(chunk):
    """Plumbing workload (f32, d=64): the first chunk (no cache) and one with a full cache."""
    wl = W.WORKLOADS[1]
    st = _state_after(wl, chunk)
    check_backward(wl, st, W.chunk_inputs(wl, 0, chunk), seed=chunk, where=f"chunk {chunk}:")


@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("chunk", [0, 5])
def test_backward_bf16_reduced(head_dim, chunk):
    """B=2, 8q/2kv heads, N_C=512, S=128: an empty cache and a full one (several tiles,
    partial diagonal tiles, G = 4 rows per position)."""
    wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=head_dim, capacity=512,
                    recent_window=64, chunk=128, seq_len=2048, heavy_count=20)
    st = _state_after(wl, chunk)
    check_backward(wl, st, W.chunk_inputs(wl, 0, chunk), seed=chunk, where=f"chunk {chunk}:")


@pytest.mark.parametrize("case", [
    dict(dtype="bf16", head_dim=64, n_q_heads=6, n_kv_heads=2, capacity=300, chunk=100,
         recent_window=10, seq_len=700),
    dict(dtype="bf16", head_dim=128, n_q_heads=3, n_kv_heads=3, capacity=97, chunk=33,
         recent_window=5, seq_len=330),
    dict(dtype="f32", head_dim=128, n_q_heads=4, n_kv_heads=2, capacity=150, chunk=65,
         recent_window=7, seq_len=520),
], ids=["bf16_d64_g3_S100", "bf16_mha_S33", "f32_d128_S65"])
def test_backward_ragged(case):
    """Ragged chunks and capacities, GQA 3 and MHA, after a few chunks."""
    wl = W.workload(2, batch=2, heavy_count=4, sm_scale=case["head_dim"] ** -0.5, **case)
    st = _state_after(wl, 4)
    check_backward(wl, st, W.chunk_inputs(wl, 0, 4), seed=4)


def test_backward_buffer_form():
    """Backward of the buffer form: the overwritten slots are not keys, gradient 0."""
    wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, capacity=512, recent_window=64,
                    chunk=128, seq_len=2048, heavy_count=20)
    st = _state_after(wl, 6)
    x = W.chunk_inputs(wl, 0, 6)
    victims = oracle.select_victims(st, wl.chunk, wl.recent_window)
    targets = np.stack([np.stack([np.sort(np.concatenate(
        [victims[b, g], np.arange(st.n, min(st.capacity, st.n + wl.chunk))]))
        for g in range(wl.n_kv_heads)]) for b in range(wl.batch)])
    check_backward(wl, st, x, seed=6, freed=targets)


def test_backward_full_size_steady():
    """Chunk 1k from a full 8192-slot cache (Qwen3-4B attention shape)."""
    wl = W.WORKLOADS[2]
    s = W.steady_state(wl, 0, start=16 * wl.chunk)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    check_backward(wl, st, W.chunk_inputs(wl, 0, 16), seed=16)


def test_backward_full_size_deterministic():
    """At the full chunk-1k shape the dK/dV rows of each key block go in two halves that
    add into zeroed buffers; two runs give the same bits (two additions to zero commute)."""
    wl = W.WORKLOADS[2]
    s = W.steady_state(wl, 0, start=16 * wl.chunk)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    dt = H.TORCH_DT[wl.dtype]
    cache = h2o.H2OCache(H.dims_of(wl), H.DEV)
    H.load_oracle_state(cache, st, wl.dtype)
    x = W.chunk_inputs(wl, 0, 16)
    q, k, v = H.dev(x["q"], dt), H.dev(x["k"], dt), H.dev(x["v"], dt)
    out, lse, _, _ = h2o.chunk_attn(cache, st.P, q, k, v, wl.sm_scale, summed_weights=False)
    dout = H.dev(_dout(wl, wl.chunk, 3), dt)
    runs = [h2o.chunk_attn_backward(cache, st.P, q, k, v, out, lse, dout, wl.sm_scale)
            for _ in range(2)]
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, *runs):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_backward_positions_outside_chunk_start(dtype, head_dim):
    """A cache whose filled slots include empty-marked slots (never visible) and slots
    holding tokens at or after the chunk start (visible from their position on): the
    backward applies the forward's positional mask."""
    wl = W.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=head_dim, capacity=500,
                    recent_window=64, chunk=128, seq_len=4096, heavy_count=20, dtype=dtype,
                    sm_scale=head_dim ** -0.5)
    s = W.steady_state(wl, 0, start=20 * wl.chunk, seed=4)
    n = wl.capacity - 37
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], n, s["start"])
    st.pos[:, :, n:] = -1
    r = np.random.default_rng(12)
    for b in range(wl.batch):
        for g in range(wl.n_kv_heads):
            idx = r.choice(n, 40, replace=False)
            st.pos[b, g, idx[:20]] = -1
            st.pos[b, g, idx[20:]] = st.P + r.integers(0, wl.chunk + 64, 20)
    check_backward(wl, st, W.chunk_inputs(wl, 0, 20), seed=3, where="positions")


def test_backward_max_capacity():
    """Chunk 1k from a full cache at the largest capacity (32768 slots, 4 query heads on
    one KV head): 512 cache key tiles per dQ block and 256 key blocks for dK/dV."""
    wl = W.workload(2, batch=1, n_q_heads=4, n_kv_heads=1, capacity=32768, recent_window=512,
                    chunk=1024, seq_len=65536)
    s = W.steady_state(wl, 0, start=40 * wl.chunk)
    st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
    check_backward(wl, st, W.chunk_inputs(wl, 0, 40), seed=40)
