"""Checks that pin the fp64 oracle to things other than itself.

Each ``check_*`` takes the oracle module as its argument so the same checks
can be run against deliberately broken copies of it (tests/test_oracle.py,
``test_planted_mistakes_are_caught``).  They raise AssertionError on failure.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "h2o_worked_examples.json")


# ----------------------------------------------------------------------------- helpers
def _val(x) -> float:
    if isinstance(x, str):
        if x.startswith("ln "):
            return math.log(float(Fraction(x[3:])))
        return float(Fraction(x))
    return float(x)


def _vals(xs):
    return np.array([[_val(y) for y in x] if isinstance(x, list) else _val(x) for x in xs],
                    dtype=np.float64)


def random_problem(seed, B=2, Hq=4, Hkv=2, d=16, N=40):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, N, d))
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d))
    return q, k, v


def run_chain(orc, q, k, v, S, NC, W, sm_scale, score_mode="h2o", state=None):
    """Feed a whole sequence through the oracle in chunks of S (last chunk may be shorter)."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    st = state if state is not None else orc.H2OState.empty(B, Hkv, NC, d)
    steps = []
    for c0 in range(0, N, S):
        c1 = min(N, c0 + S)
        steps.append(orc.h2o_step(st, q[:, :, c0:c1], k[:, :, c0:c1], v[:, :, c0:c1],
                                  sm_scale, W, score_mode))
    return st, steps


def exact_causal_sdpa(q, k, v, sm_scale):
    """Full causal GQA attention from torch's SDPA in fp64 on the CPU."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, G, axis=1))
    vt = torch.from_numpy(np.repeat(v, G, axis=1))
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=sm_scale).numpy()


def exact_causal_weights(q, k, sm_scale):
    """The attention matrix itself: SDPA with an identity value matrix returns it."""
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    eye = torch.eye(N, dtype=torch.float64).expand(B, Hq, N, N)
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, G, axis=1))
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, eye, is_causal=True, scale=sm_scale).numpy()


# ------------------------------------------------------------------------------ checks
def check_golden(orc):
    """Hand-derived worked examples (tests/golden/h2o_worked_examples.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        dims, st, ch, ex = case["dims"], case["state"], case["chunk"], case["expect"]
        NC = dims["capacity"]
        state = orc.H2OState.from_arrays(
            np.array(st["k"], np.float64).reshape(1, 1, NC, 1),
            np.array(st["v"], np.float64).reshape(1, 1, NC, 1),
            np.array(st["pos"]).reshape(1, 1, NC),
            _vals(st["phi"]).reshape(1, 1, NC), st["n"], st["P"])
        S = len(ch["k"])
        Hq = dims["Hq"]
        q = np.array(ch["q"], np.float64).reshape(1, Hq, S, 1)
        kn = np.array(ch["k"], np.float64).reshape(1, 1, S, 1)
        vn = np.array(ch["v"], np.float64).reshape(1, 1, S, 1)
        res = orc.h2o_step(state, q, kn, vn, dims["sm_scale"], dims["W"],
                           dims.get("score_mode", "h2o"))
        name = case["name"]
        np.testing.assert_allclose(res["out"].reshape(-1), _vals(ex["out"]).reshape(-1),
                                   rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(res["lse"].reshape(-1), _vals(ex["lse"]),
                                   rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(res["colsum_cache"].reshape(-1), _vals(ex["colsum_cache"]),
                                   rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(res["colsum_new"].reshape(-1), _vals(ex["colsum_new"]),
                                   rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(res["phi_updated"].reshape(-1), _vals(ex["phi_updated"]),
                                   rtol=0, atol=1e-12, err_msg=name)
        assert res["freed_slots"].reshape(-1).tolist() == ex["freed_slots"], name
        assert state.pos.reshape(-1).tolist() == ex["pos_after"], name
        np.testing.assert_allclose(state.phi.reshape(-1), _vals(ex["phi_after"]),
                                   rtol=0, atol=1e-12, err_msg=name)
        assert state.n == ex["n_after"] and state.P == ex["P_after"], name


def check_rows_normalised(orc, seed=1):
    """V = 1 gives out = 1 (each row's weights sum to 1); summed weights total S*G."""
    q, k, v = random_problem(seed, N=48)
    NC, S, W = 24, 8, 4
    ones = np.ones_like(v)
    st, steps = run_chain(orc, q, k, ones, S, NC, W, 0.3)
    G = q.shape[1] // k.shape[1]
    for res in steps:
        np.testing.assert_allclose(res["out"], 1.0, rtol=0, atol=1e-12)
        tot = res["colsum_cache"].sum(axis=2) + res["colsum_new"].sum(axis=2)
        np.testing.assert_allclose(tot, res["out"].shape[2] * G, rtol=1e-12)


def check_exact_when_no_eviction(orc, seed=2, S=8):
    """Capacity >= sequence: output equals torch SDPA causal attention of the whole sequence,
    lse equals torch.logsumexp of the causal logits, and the final scores equal the column
    sums of the full causal attention matrix (SDPA with V = identity)."""
    q, k, v = random_problem(seed, N=40)
    sm = 0.37
    N = q.shape[2]
    st, steps = run_chain(orc, q, k, v, S, NC=64, W=3, sm_scale=sm)
    out = np.concatenate([r["out"] for r in steps], axis=2)
    lse = np.concatenate([r["lse"] for r in steps], axis=2)
    np.testing.assert_allclose(out, exact_causal_sdpa(q, k, v, sm), rtol=0, atol=1e-12)
    G = q.shape[1] // k.shape[1]
    logits = torch.from_numpy(q) @ torch.from_numpy(np.repeat(k, G, axis=1)).transpose(-1, -2)
    logits = logits * sm
    logits = logits.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)
    A = exact_causal_weights(q, k, sm)                                # (B, Hq, N, N)
    B, Hq = q.shape[:2]
    colsum = A.sum(axis=2).reshape(B, Hq // G, G, N).sum(axis=2)    # sum over rows, group
    assert st.n == N
    phi_by_pos = np.zeros_like(colsum)
    for b in range(B):
        for g in range(colsum.shape[1]):
            phi_by_pos[b, g, st.pos[b, g, :N]] = st.phi[b, g, :N]
    np.testing.assert_allclose(phi_by_pos, colsum, rtol=1e-12, atol=1e-12)


def check_large_logits(orc, seed=15, S=8):
    """Logits in the thousands (queries scaled by 300): with each row's maximum taken out
    before the exponentials, output and lse still equal torch's fp64 SDPA and logsumexp of
    the causal logits; without it the exponentials overflow."""
    q, k, v = random_problem(seed, N=40)
    q = q * 300.0
    sm = 0.37
    N = q.shape[2]
    st, steps = run_chain(orc, q, k, v, S, NC=64, W=3, sm_scale=sm)
    out = np.concatenate([r["out"] for r in steps], axis=2)
    lse = np.concatenate([r["lse"] for r in steps], axis=2)
    G = q.shape[1] // k.shape[1]
    logits = torch.from_numpy(q) @ torch.from_numpy(np.repeat(k, G, axis=1)).transpose(-1, -2)
    logits = (logits * sm).masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    want_lse = torch.logsumexp(logits, dim=-1).numpy()
    assert np.abs(want_lse).max() > 1000, "logits not large enough for this check"
    np.testing.assert_allclose(out, exact_causal_sdpa(q, k, v, sm), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-13, atol=0)


def check_chunk_size_invariance(orc, seed=3):
    """Without eviction the results do not depend on the chunk length (1, 7, 16)."""
    q, k, v = random_problem(seed, N=32)
    ref = None
    for S in (1, 7, 16):
        st, steps = run_chain(orc, q, k, v, S, NC=32, W=0, sm_scale=0.5)
        out = np.concatenate([r["out"] for r in steps], axis=2)
        phi = np.take_along_axis(st.phi, np.argsort(st.pos, axis=2), axis=2)
        if ref is None:
            ref = (out, phi)
        else:
            np.testing.assert_allclose(out, ref[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(phi, ref[1], rtol=1e-12, atol=1e-12)


def check_uniform_closed_form(orc):
    """q = 0: uniform causal attention.  Output i = mean of v[0..i]; with no eviction the
    score of position j is G * sum_{i=j}^{N-1} 1/(i+1)."""
    B, Hq, Hkv, d, N = 1, 6, 2, 3, 30
    G = Hq // Hkv
    r = np.random.default_rng(4)
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d))
    q = np.zeros((B, Hq, N, d))
    st, steps = run_chain(orc, q, k, v, S=4, NC=N, W=0, sm_scale=1.0)
    out = np.concatenate([r_["out"] for r_ in steps], axis=2)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(out, np.repeat(prefix_mean, G, axis=1), rtol=0, atol=1e-12)
    tail = np.array([sum(1.0 / (i + 1) for i in range(j, N)) for j in range(N)])
    for g in range(Hkv):
        np.testing.assert_allclose(st.phi[0, g, st.pos[0, g] >= 0][np.argsort(st.pos[0, g])],
                                   G * tail, rtol=1e-12)


def _k_smallest_bruteforce(phi, eligible, k):
    """Among all k-subsets of the eligible slots, the one whose sorted (phi, slot) list is
    lexicographically smallest; it also has the smallest phi sum."""
    best = None
    for sub in itertools.combinations(eligible, k):
        key = sorted((phi[j], j) for j in sub)
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(best[1]), sum(phi[j] for j in best[1])


def check_bruteforce_selection(orc, trials=150):
    """Tiny caches (N_C <= 6, S <= 2, W <= 2): the victim set is the lexicographically
    smallest (phi, slot) k-subset of the eligible slots, found by enumeration."""
    r = np.random.default_rng(5)
    for t in range(trials):
        NC = int(r.integers(2, 7))
        S = int(r.integers(1, 3))
        W = int(r.integers(0, 3))
        n = NC
        P = NC + int(r.integers(0, 4))
        pos = r.permutation(P)[:NC]
        phi = r.integers(0, 3, NC).astype(np.float64) / 2.0      # many exact ties
        st = orc.H2OState.from_arrays(np.zeros((1, 1, NC, 1)), np.zeros((1, 1, NC, 1)),
                                      pos.reshape(1, 1, NC), phi.reshape(1, 1, NC), n, P)
        k = max(0, n + S - NC)
        eligible = [j for j in range(n) if pos[j] < P - W]
        if len(eligible) < k:
            try:
                orc.select_victims(st, S, W)
            except ValueError:
                continue
            raise AssertionError("capacity shortfall not reported")
        got = orc.select_victims(st, S, W)[0, 0].tolist()
        want, want_sum = _k_smallest_bruteforce(phi, eligible, k)
        assert got == want, (t, got, want, phi, pos, W, P)
        assert sum(phi[j] for j in got) == want_sum
        # the minimum phi sum over all k-subsets is achieved
        if k:
            best_sum = min(sum(phi[j] for j in sub)
                           for sub in itertools.combinations(eligible, k))
            assert want_sum == best_sum


def check_decode_is_argmin(orc, trials=50):
    """S = 1: the single victim is numpy's argmin over the eligible scores (first index on ties)."""
    r = np.random.default_rng(6)
    for _ in range(trials):
        NC, W = 9, 2
        P = 20
        pos = r.permutation(P)[:NC]
        phi = r.integers(0, 4, NC).astype(np.float64)
        st = orc.H2OState.from_arrays(np.zeros((1, 1, NC, 1)), np.zeros((1, 1, NC, 1)),
                                      pos.reshape(1, 1, NC), phi.reshape(1, 1, NC), NC, P)
        elig = np.where(pos < P - W)[0]
        want = elig[np.argmin(phi[elig])]
        assert orc.select_victims(st, 1, W)[0, 0].tolist() == [want]


def check_dense_masked_replay(orc, seed=7):
    """Replay the chain over the full token history: every chunk recomputed with a dense
    mask built only from the freed-slot log must reproduce the slot-based outputs; scores
    rebuilt from those column sums must pick the same victims."""
    B, Hq, Hkv, d, N = 1, 4, 2, 8, 44
    S, NC, W, sm = 4, 12, 2, 0.8
    G = Hq // Hkv
    q, k, v = random_problem(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N)
    st, steps = run_chain(orc, q, k, v, S, NC, W, sm)
    slot_tok = np.full((B, Hkv, NC), -1)        # token held by each slot, from the log only
    phi_tok = np.zeros((B, Hkv, N))             # score per token, rebuilt from replay
    for c, res in enumerate(steps):
        c0, c1 = c * S, min(N, c * S + S)
        for b in range(B):
            for g in range(Hkv):
                resident = [t for t in slot_tok[b, g] if t >= 0]
                keys = resident + list(range(c0, c1))
                summed = np.zeros(len(keys))
                for hh in range(G):
                    h = g * G + hh
                    s = sm * q[b, h, c0:c1] @ k[b, g, keys].T
                    mask = np.array(keys)[None, :] <= np.arange(c0, c1)[:, None]
                    s = np.where(mask, s, -np.inf)
                    w = torch.softmax(torch.from_numpy(s), dim=-1).numpy()
                    np.testing.assert_allclose(res["out"][b, h], w @ v[b, g, keys],
                                               rtol=0, atol=1e-12)
                    summed += w.sum(axis=0)
                for t, cs in zip(keys, summed):
                    phi_tok[b, g, t] += cs
                # colsum_cache reported per slot maps to the resident tokens
                for j in range(NC):
                    if slot_tok[b, g, j] >= 0:
                        np.testing.assert_allclose(
                            res["colsum_cache"][b, g, j],
                            summed[keys.index(slot_tok[b, g, j])], rtol=1e-12, atol=1e-15)
                # expected victims from the rebuilt scores
                n_before = int((slot_tok[b, g] >= 0).sum())
                kk = max(0, n_before + (c1 - c0) - NC)
                elig = [j for j in range(n_before) if slot_tok[b, g, j] < c0 - W]
                order = sorted(elig, key=lambda j: (phi_tok[b, g, slot_tok[b, g, j]], j))
                assert sorted(order[:kk]) == res["victims"][b, g].tolist()
                targets = sorted(order[:kk] + list(range(n_before, min(NC, n_before + c1 - c0))))
                assert res["freed_slots"][b, g].tolist() == targets
                for i, j in enumerate(targets):
                    slot_tok[b, g, j] = c0 + i
    assert (st.pos == slot_tok).all()


def check_conservation_and_monotonicity(orc, seed=8):
    """Resident scores plus scores at eviction add up to G * rows processed; a resident
    slot's score never decreases."""
    q, k, v = random_problem(seed, N=60)
    G = q.shape[1] // k.shape[1]
    S, NC, W = 6, 18, 3
    B, Hq, N, d = q.shape
    st = orc.H2OState.empty(B, k.shape[1], NC, d)
    evicted = np.zeros((B, k.shape[1]))
    prev_phi, prev_pos = None, None
    for c0 in range(0, N, S):
        res = orc.h2o_step(st, q[:, :, c0:c0 + S], k[:, :, c0:c0 + S], v[:, :, c0:c0 + S],
                           0.6, W)
        if prev_phi is not None:
            same = (st.pos == prev_pos) & (prev_pos >= 0)
            assert (st.phi[same] >= prev_phi[same]).all()
        evicted += res["evicted_phi"].sum(axis=2)
        total = st.phi[:, :, :st.n].sum(axis=2) + evicted
        np.testing.assert_allclose(total, G * (c0 + S), rtol=1e-12)
        prev_phi, prev_pos = st.phi.copy(), st.pos.copy()


def check_slot_permutation_invariance(orc, seed=9):
    """Permuting the slots of a full cache (K, V, t, phi together) leaves out and lse
    unchanged, permutes the summed weights, and maps the victims accordingly."""
    r = np.random.default_rng(seed)
    B, Hq, Hkv, d, NC, S, W, P = 1, 4, 2, 8, 16, 4, 3, 40
    K = r.standard_normal((B, Hkv, NC, d))
    V = r.standard_normal((B, Hkv, NC, d))
    pos = np.stack([np.stack([np.sort(r.choice(P, NC, replace=False)) for _ in range(Hkv)])])
    phi = r.random((B, Hkv, NC)) * 5
    q = r.standard_normal((B, Hq, S, d))
    kn = r.standard_normal((B, Hkv, S, d))
    vn = r.standard_normal((B, Hkv, S, d))
    perm = r.permutation(NC)
    a = orc.H2OState.from_arrays(K, V, pos, phi, NC, P)
    b = orc.H2OState.from_arrays(K[:, :, perm], V[:, :, perm], pos[:, :, perm],
                                 phi[:, :, perm], NC, P)
    ra = orc.h2o_step(a, q, kn, vn, 0.4, W)
    rb = orc.h2o_step(b, q, kn, vn, 0.4, W)
    np.testing.assert_allclose(ra["out"], rb["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ra["lse"], rb["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ra["colsum_cache"][:, :, perm], rb["colsum_cache"],
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ra["colsum_new"], rb["colsum_new"], rtol=1e-12)
    for g in range(Hkv):
        va = sorted(ra["victims"][0, g].tolist())
        vb = sorted(perm[rb["victims"][0, g]].tolist())
        assert va == vb


def lastrec_resident(c0, NC, beta):
    """Closed form of the lastrec cache before the chunk starting at token c0: every
    earlier token while they fit, else the first beta and the last NC - beta."""
    if c0 <= NC:
        return list(range(c0))
    return list(range(beta)) + list(range(c0 - (NC - beta), c0))


def check_lastrec_closed_form(orc, seed=10):
    """lastrec keeps the first beta and the last N_C - beta tokens: the cache holds that
    set after every chunk, K and V rows follow their tokens, and every chunk's output is
    torch's SDPA over exactly those keys plus the chunk's causal keys."""
    B, Hq, Hkv, d, N = 2, 4, 2, 8, 53
    G = Hq // Hkv
    sm = 0.7
    q, k, v = random_problem(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N)
    for S, NC, beta in [(4, 16, 3), (5, 12, 0), (3, 10, 7), (1, 9, 2)]:
        st = orc.H2OState.empty(B, Hkv, NC, d)
        for c0 in range(0, N, S):
            c1 = min(N, c0 + S)
            keys = lastrec_resident(c0, NC, beta) + list(range(c0, c1))
            res = orc.lastrec_step(st, q[:, :, c0:c1], k[:, :, c0:c1], v[:, :, c0:c1], sm, beta)
            kk = torch.from_numpy(np.repeat(k[:, :, keys], G, axis=1))
            vv = torch.from_numpy(np.repeat(v[:, :, keys], G, axis=1))
            mask = torch.from_numpy(np.array(keys)[None, :] <= np.arange(c0, c1)[:, None])
            want = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[:, :, c0:c1]), kk, vv, attn_mask=mask, scale=sm).numpy()
            np.testing.assert_allclose(res["out"], want, rtol=0, atol=1e-12)
            held = sorted(lastrec_resident(c1, NC, beta))
            for b in range(B):
                for g in range(Hkv):
                    assert sorted(st.pos[b, g, :st.n].tolist()) == held
                    np.testing.assert_array_equal(st.K[b, g, :st.n], k[b, g, st.pos[b, g, :st.n]])
                    np.testing.assert_array_equal(st.V[b, g, :st.n], v[b, g, st.pos[b, g, :st.n]])
                    assert res["freed_slots"][b, g].tolist() == sorted(res["freed_slots"][b, g])


def check_lastrec_capacity_error(orc):
    """lastrec cannot evict the first beta tokens: a chunk longer than N_C - beta into a
    full cache has too few eligible slots and must be refused."""
    NC, beta, d = 8, 5, 4
    st = orc.H2OState.empty(1, 1, NC, d)
    z = np.zeros((1, 1, NC, d))
    orc.lastrec_step(st, z, z, z, 1.0, beta)               # fills the cache
    z4 = np.zeros((1, 1, 4, d))
    try:
        orc.lastrec_step(st, z4, z4, z4, 1.0, beta)        # needs 4 of 3 eligible
    except ValueError:
        return
    raise AssertionError("lastrec accepted more victims than eligible slots")


def check_buffer_without_eviction_is_attend_first(orc, seed=11):
    """While nothing is evicted the two orders see the same keys: the buffer form gives
    the outputs, log-sum-exps, positions and scores of the attend-first step."""
    q, k, v = random_problem(seed, N=30)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    a = orc.H2OState.empty(B, Hkv, 32, d)
    b = orc.H2OState.empty(B, Hkv, 32, d)
    for c0 in range(0, N, 7):
        x = (q[:, :, c0:c0 + 7], k[:, :, c0:c0 + 7], v[:, :, c0:c0 + 7])
        ra = orc.h2o_step(a, *x, 0.5, 3)
        rb = orc.buffer_step(b, *x, 0.5, 3)
        np.testing.assert_allclose(rb["out"], ra["out"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(rb["lse"], ra["lse"], rtol=0, atol=1e-12)
        assert (a.pos == b.pos).all()
        np.testing.assert_allclose(b.phi, a.phi, rtol=1e-12, atol=1e-15)


def check_buffer_dense_replay(orc, seed=12):
    """Replay the buffer form over the full token history: every chunk recomputed with
    torch's fp64 SDPA under a mask built only from the freed-slot log (the resident tokens
    after insertion, causal by position) must give the slot-based outputs, and scores
    rebuilt from those weights -- before the chunk -- must pick the same victims."""
    B, Hq, Hkv, d, N = 1, 4, 2, 8, 44
    S, NC, W, sm = 4, 12, 2, 0.8
    G = Hq // Hkv
    q, k, v = random_problem(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N)
    st = orc.H2OState.empty(B, Hkv, NC, d)
    slot_tok = np.full((B, Hkv, NC), -1)
    phi_tok = np.zeros((B, Hkv, N))
    for c0 in range(0, N, S):
        c1 = min(N, c0 + S)
        res = orc.buffer_step(st, q[:, :, c0:c1], k[:, :, c0:c1], v[:, :, c0:c1], sm, W)
        for b in range(B):
            for g in range(Hkv):
                n_before = int((slot_tok[b, g] >= 0).sum())
                kk = max(0, n_before + (c1 - c0) - NC)
                elig = [j for j in range(n_before) if slot_tok[b, g, j] < c0 - W]
                order = sorted(elig, key=lambda j: (phi_tok[b, g, slot_tok[b, g, j]], j))
                assert sorted(order[:kk]) == res["victims"][b, g].tolist()
                targets = sorted(order[:kk] + list(range(n_before, min(NC, n_before + c1 - c0))))
                assert res["freed_slots"][b, g].tolist() == targets
                for i, j in enumerate(targets):
                    slot_tok[b, g, j] = c0 + i
                keys = [int(t) for t in slot_tok[b, g] if t >= 0]
                mask = torch.from_numpy(np.array(keys)[None, :] <= np.arange(c0, c1)[:, None])
                for hh in range(G):
                    h = g * G + hh
                    qt = torch.from_numpy(q[b, h, c0:c1])
                    kt = torch.from_numpy(k[b, g, keys])
                    want = torch.nn.functional.scaled_dot_product_attention(
                        qt, kt, torch.from_numpy(v[b, g, keys]), attn_mask=mask, scale=sm).numpy()
                    np.testing.assert_allclose(res["out"][b, h], want, rtol=0, atol=1e-12)
                    w = torch.nn.functional.scaled_dot_product_attention(
                        qt, kt, torch.eye(len(keys), dtype=torch.float64), attn_mask=mask,
                        scale=sm).numpy()
                    for t, cs in zip(keys, w.sum(axis=0)):
                        phi_tok[b, g, t] += cs
    for b in range(B):
        for g in range(Hkv):
            for j in range(NC):
                if slot_tok[b, g, j] >= 0:
                    np.testing.assert_allclose(st.phi[b, g, j], phi_tok[b, g, slot_tok[b, g, j]],
                                               rtol=1e-12, atol=1e-15)


def check_backward_is_autograd(orc, seed=13):
    """The gradients equal torch autograd through fp64 SDPA over the same keys under the
    same mask: the filled slots (some excluded) and the chunk's causal keys."""
    r = np.random.default_rng(seed)
    B, Hq, Hkv, d, NC, n, S, P = 2, 4, 2, 8, 24, 17, 6, 30
    G = Hq // Hkv
    K = r.standard_normal((B, Hkv, NC, d))
    V = r.standard_normal((B, Hkv, NC, d))
    pos = np.stack([np.stack([np.sort(r.choice(P, NC, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)])
    st = orc.H2OState.from_arrays(K, V, pos, np.zeros((B, Hkv, NC)), n, P)
    q = r.standard_normal((B, Hq, S, d))
    kn = r.standard_normal((B, Hkv, S, d))
    vn = r.standard_normal((B, Hkv, S, d))
    dout = r.standard_normal((B, Hq, S, d))
    excl = r.random((B, Hkv, NC)) < 0.25
    sm = 0.45
    got = orc.attend_chunk_backward(st, q, kn, vn, dout, sm, excluded=excl)
    qt = torch.from_numpy(q).requires_grad_()
    kc = torch.from_numpy(K[:, :, :n].copy()).requires_grad_()
    vc = torch.from_numpy(V[:, :, :n].copy()).requires_grad_()
    knt = torch.from_numpy(kn).requires_grad_()
    vnt = torch.from_numpy(vn).requires_grad_()
    keys = torch.cat([kc, knt], dim=2).repeat_interleave(G, dim=1)
    vals = torch.cat([vc, vnt], dim=2).repeat_interleave(G, dim=1)
    t = np.concatenate([pos[:, :, :n], np.broadcast_to(P + np.arange(S), (B, Hkv, S))], axis=2)
    vis = (t[:, :, None, :] <= (P + np.arange(S))[None, None, :, None])
    vis[:, :, :, :n] &= ~excl[:, :, None, :n]
    mask = torch.from_numpy(np.repeat(vis, G, axis=1))
    out = torch.nn.functional.scaled_dot_product_attention(qt, keys, vals, attn_mask=mask, scale=sm)
    out.backward(torch.from_numpy(dout))
    want = [qt.grad, knt.grad, vnt.grad, kc.grad, vc.grad]
    for gi, wi in zip(got[:3], want[:3]):
        np.testing.assert_allclose(gi, wi.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got[3][:, :, :n], want[3].numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got[4][:, :, :n], want[4].numpy(), rtol=1e-9, atol=1e-11)
    assert (got[3][:, :, n:] == 0).all() and (got[4][:, :, n:] == 0).all()
    assert (got[3][excl & (np.arange(NC) < n)] == 0).all()


def check_backward_finite_differences(orc, seed=14):
    """Central differences of L = sum(O * dO) on a tiny case match the gradients."""
    r = np.random.default_rng(seed)
    B, Hq, Hkv, d, NC, n, S, P = 1, 2, 1, 3, 5, 4, 3, 7
    K = r.standard_normal((B, Hkv, NC, d))
    V = r.standard_normal((B, Hkv, NC, d))
    pos = np.array([[[0, 2, 5, 6, -1]]])
    q = r.standard_normal((B, Hq, S, d))
    kn = r.standard_normal((B, Hkv, S, d))
    vn = r.standard_normal((B, Hkv, S, d))
    dout = r.standard_normal((B, Hq, S, d))
    sm = 0.7

    def loss(K_, V_, q_, kn_, vn_):
        st = orc.H2OState.from_arrays(K_, V_, pos, np.zeros((B, Hkv, NC)), n, P)
        return (orc.attend_chunk(st, q_, kn_, vn_, sm)[0] * dout).sum()
    st = orc.H2OState.from_arrays(K, V, pos, np.zeros((B, Hkv, NC)), n, P)
    got = orc.attend_chunk_backward(st, q, kn, vn, dout, sm)
    args = [K, V, q, kn, vn]
    names = {2: 0, 3: 1, 4: 2, 0: 3, 1: 4}          # argument -> index in got
    eps = 1e-6
    for ai, arr in enumerate(args):
        g = got[names[ai]]
        for idx in np.ndindex(arr.shape):
            if ai in (0, 1) and idx[2] >= n:
                continue
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[ai][idx] += eps
            minus[ai][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (ai, idx, fd, g[idx])


ALL_CHECKS = [check_golden, check_rows_normalised, check_exact_when_no_eviction,
              check_large_logits,
              check_chunk_size_invariance, check_uniform_closed_form,
              check_bruteforce_selection, check_decode_is_argmin, check_dense_masked_replay,
              check_conservation_and_monotonicity, check_slot_permutation_invariance,
              check_lastrec_closed_form, check_lastrec_capacity_error,
              check_buffer_without_eviction_is_attend_first, check_buffer_dense_replay,
              check_backward_is_autograd, check_backward_finite_differences]
