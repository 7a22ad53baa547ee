"""Seeded generators: determinism, bf16 rounding, and the workload recipes (CPU only)."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.4e38], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (W.bf16_bits(x) == want).all()
    np.testing.assert_array_equal(W.bf16_round(x),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_chunks_are_deterministic_and_independent():
    wl = W.workload(2, seq_len=4096, capacity=1024, chunk=512, heavy_count=41)
    a = W.chunk_inputs(wl, 0, 3)
    b = W.chunk_inputs(wl, 0, 3)
    c = W.chunk_inputs(wl, 0, 4)
    for key in ("q", "k", "v"):
        assert (a[key] == b[key]).all()
        assert not (a[key] == c[key]).all()
        assert a[key].dtype == np.float32
        assert (W.bf16_round(a[key]) == a[key]).all()      # bf16-exact
    assert a["q"].shape == (1, 32, 512, 128) and a["k"].shape == (1, 8, 512, 128)


def test_heavy_positions_boosted():
    wl = W.workload(2, seq_len=8192, capacity=1024, chunk=1024, heavy_count=82)
    hpos, hdir = W.heavy_boost(wl, 0)
    assert hpos.shape == (1, 82) and np.allclose(np.linalg.norm(hdir, axis=1), 1, atol=1e-6)
    c = int(hpos[0, 0] // wl.chunk)
    x = W.chunk_inputs(wl, 0, c)
    t = int(hpos[0, 0] - c * wl.chunk)
    proj = x["k"][0, :, t, :] @ hdir[0]
    others = x["k"][0, :, (t + 1) % wl.chunk, :] @ hdir[0]
    assert (proj > 2.0 - 4.5).all() and abs(proj.mean() - others.mean()) > 0.5


def test_plumbing_query_mean_direction():
    wl = W.WORKLOADS[1]
    hpos, hdir = W.heavy_boost(wl, 0)
    qs = np.concatenate([W.chunk_inputs(wl, 0, c)["q"] for c in range(wl.n_chunks)], axis=2)
    u = qs.astype(np.float64).mean(axis=(1, 2))[0]
    np.testing.assert_allclose(hdir[0], u / np.linalg.norm(u), atol=1e-6)
    assert hpos.shape == (1, 8)


def test_steady_state_shape_and_positions():
    wl = W.workload(2, capacity=2048, chunk=256)
    st = W.steady_state(wl, 0, start=8192, seed=1)
    pos = st["pos"]
    assert pos.shape == (1, 8, 2048) and pos.dtype == np.int32
    for g in range(8):
        assert len(set(pos[0, g].tolist())) == 2048
        assert pos[0, g].max() < 8192 and pos[0, g].min() >= 0
        assert set(range(8192 - 256, 8192)) <= set(pos[0, g].tolist())
    assert (st["phi"] > 0).all()


def test_decode_initial_state():
    wl = W.workload(5, capacity=512, seq_len=8, batch=2)
    st = W.decode_initial_state(wl)
    assert st["k"].shape == (2, 8, 512, 128)
    assert (st["pos"][1, 3] == np.arange(512)).all()
    tail = np.cumsum((1.0 / np.arange(1, 513))[::-1])[::-1]
    jitter = np.log(st["phi"] / (wl.group * tail))
    assert abs(jitter.mean()) < 0.02 and abs(jitter.std() - 0.25) < 0.02
    x = W.decode_step_inputs(wl, 3)
    assert x["q"].shape == (2, 32, 1, 128) and x["start"] == 515


def test_layer_stack_layers_draw_independently():
    """The 36-layer stack: each layer has its own inputs, heavy positions and cache state."""
    wl = W.workload(4, seq_len=8192, capacity=1024, chunk=256, heavy_count=82)
    assert W.WORKLOADS[4].layers == 36
    a, b = W.chunk_inputs(wl, 0, 2), W.chunk_inputs(wl, 35, 2)
    for key in ("q", "k", "v"):
        assert a[key].shape == b[key].shape
        assert np.corrcoef(a[key].ravel(), b[key].ravel())[0, 1] < 0.05
    ha, hb = W.heavy_boost(wl, 0)[0], W.heavy_boost(wl, 35)[0]
    assert not np.array_equal(ha, hb)
    sa, sb = W.steady_state(wl, 0, start=2048), W.steady_state(wl, 35, start=2048)
    assert not np.array_equal(sa["pos"], sb["pos"]) and not np.array_equal(sa["k"], sb["k"])
