"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare
it with the fp64 oracle on identical seeded inputs.

Tolerances (bf16): attention output |got - ref| <= 1e-2 + halfulp(ref) per
element, where halfulp(ref) is half a bf16 ulp of the reference value (the
rounding that storing the output in bf16 costs by itself), and relative L2
<= 5e-3; log-sum-exp abs <= 1e-3; summed weights and scores relative <= 1e-3.
The number of elements above the flat 1e-2 is printed for every comparison.
(f32): output |got - ref| <= 1e-4 + halfulp_f32(ref), relative L2 <= 1e-5,
lse abs <= 1e-5, summed weights and scores relative <= 1e-5.

Victim sets must match exactly, except that a swap of two slots straddling the
cut is accepted when their oracle ranking values (the score, or for h2o-norm
the score over the age, both in fp64) are within 1e-5 (relative) of the cut
value; the GPU cache is then reloaded from the oracle's state so the next chunk
starts from the same input.
"""
from __future__ import annotations

import numpy as np
import torch

import h2o_sparse_attention_amd as h2o
import oracle

DEV = torch.device("cuda:0")
TOL = {
    "bf16": dict(out_abs=1e-2, mant_bits=8, out_rel_l2=5e-3, lse_abs=1e-3, cs_rel=1e-3),
    "f32": dict(out_abs=1e-4, mant_bits=24, out_rel_l2=1e-5, lse_abs=1e-5, cs_rel=1e-5),
}
NEAR_TIE_REL = 1e-5
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV, dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() \
        else t.detach().cpu().numpy()


def dims_of(wl) -> h2o.H2ODims:
    return h2o.H2ODims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity,
                       wl.recent_window, wl.dtype)


def load_oracle_state(cache: h2o.H2OCache, st: oracle.H2OState, dtype: str):
    dt = TORCH_DT[dtype]
    cache.load(dev(st.K, dt), dev(st.V, dt), dev(st.pos.astype(np.int32), torch.int32),
               dev(st.phi.astype(np.float32), torch.float32), st.n, st.P)


def gpu_chunk(cache: h2o.H2OCache, x: dict, sm_scale: float, dtype: str,
              score_mode: str = "h2o") -> dict:
    """The three calls, with a snapshot of the scores between update and eviction."""
    dt = TORCH_DT[dtype]
    q, k, v = dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt)
    P = cache.next_pos
    out, lse, cs_cache, cs_new = h2o.chunk_attn(cache, P, q, k, v, sm_scale)
    h2o.update_scores(cache, cs_cache)
    phi_upd = cache.score.clone()
    freed = h2o.evict_and_insert(cache, P, k, v, cs_new, score_mode=score_mode)
    torch.cuda.synchronize()
    return {"out": host(out), "lse": host(lse), "colsum_cache": host(cs_cache),
            "colsum_new": host(cs_new), "phi_updated": host(phi_upd),
            "freed_slots": host(freed).astype(np.int64),
            "K": cache.k.clone(), "V": cache.v.clone(), "pos": host(cache.pos).astype(np.int64),
            "phi": host(cache.score), "n": cache.n_valid}


def half_ulp(ref, dtype):
    """Half an ulp of each reference value in the storage type (bf16: 8 significand
    bits, f32: 24); 0 for 0."""
    _, e = np.frexp(np.abs(ref))            # |ref| = m 2^e, m in [0.5, 1)
    return np.where(ref != 0, np.ldexp(1.0, e - 1 - TOL[dtype]["mant_bits"]), 0.0)


def out_bound(ref, dtype):
    """Per-element bound on the attention output: the flat tolerance plus the
    output's own storage rounding."""
    return TOL[dtype]["out_abs"] + half_ulp(ref, dtype)


def check_out(g_out, r_out, dtype, where=""):
    """Per-element and relative-L2 check of an attention output; prints the worst
    element and how many exceed the flat tolerance alone."""
    tol = TOL[dtype]
    diff = np.abs(g_out - r_out)
    bound = out_bound(r_out, dtype)
    l2 = np.linalg.norm(g_out - r_out) / np.linalg.norm(r_out)
    at = np.unravel_index((diff / bound).argmax(), diff.shape)
    info = (f"worst at {tuple(int(x) for x in at)} err={diff[at]:.3e} |ref|={abs(r_out[at]):.4f} "
            f"rel-L2={l2:.2e} |ref|max={np.abs(r_out).max():.3f} "
            f"n_over_flat={(diff > tol['out_abs']).sum()} of {diff.size}")
    print(f"{where} out max-abs {diff.max():.3e} {info}")
    assert (diff <= bound).all(), f"{where} out error over bound: {info}"
    assert l2 <= tol["out_rel_l2"], f"{where} out rel-L2 {l2:.3e}"
    return diff.max(), l2


def rel_err(got, want, floor=1e-30):
    return np.abs(got - want) / np.maximum(np.abs(want), floor)


def compare_attention(g: dict, r: dict, n: int, dtype: str, where: str = ""):
    tol = TOL[dtype]
    d_out, l2 = check_out(g["out"], r["out"], dtype, where)
    d_lse = np.abs(g["lse"] - r["lse"]).max()
    assert d_lse <= tol["lse_abs"], f"{where} lse abs {d_lse:.3e}"
    e1 = rel_err(g["colsum_cache"][:, :, :n], r["colsum_cache"][:, :, :n]).max(initial=0.0)
    e2 = rel_err(g["colsum_new"], r["colsum_new"]).max()
    assert e1 <= tol["cs_rel"], f"{where} colsum_cache rel {e1:.3e}"
    assert e2 <= tol["cs_rel"], f"{where} colsum_new rel {e2:.3e}"
    assert (g["colsum_cache"][:, :, n:] == 0).all(), f"{where} colsum beyond n not zero"
    return {"out_abs": d_out, "out_l2": l2, "lse_abs": d_lse, "cs_rel": max(e1, e2)}


def compare_victims(g_freed, r_freed, r_rank, pos_before, n, P, W, where=""):
    """Returns the number of accepted near-tie swaps (0 = identical).  r_rank: the
    oracle's ranking values of the slots (fp64 score, or score over age)."""
    swaps = 0
    B, Hkv, S = r_freed.shape
    for b in range(B):
        for h in range(Hkv):
            gv = {int(x) for x in g_freed[b, h] if x < n}
            ov = {int(x) for x in r_freed[b, h] if x < n}
            assert sorted(g_freed[b, h].tolist()) == g_freed[b, h].tolist(), \
                f"{where} freed not ascending"
            assert len(set(g_freed[b, h].tolist())) == S, f"{where} freed not distinct"
            if gv == ov:
                continue
            phi = r_rank[b, h]
            cut = max(phi[j] for j in ov)
            for a in gv - ov:
                assert pos_before[b, h, a] < P - W, f"{where} evicted a protected slot {a}"
                assert phi[a] - cut <= NEAR_TIE_REL * cut, \
                    f"{where} ({b},{h}) slot {a} phi {phi[a]!r} vs cut {cut!r}"
            for o in ov - gv:
                assert cut - phi[o] <= NEAR_TIE_REL * cut, \
                    f"{where} ({b},{h}) kept slot {o} phi {phi[o]!r} vs cut {cut!r}"
            swaps += len(gv - ov)
    return swaps


def compare_rows(gk, gv, st: oracle.H2OState, slots, dtype: str, where: str = ""):
    """K / V rows of the given slots (B, Hkv, m) bit-exact against the oracle's."""
    dt = TORCH_DT[dtype]
    B, Hkv, _ = slots.shape
    for b in range(B):
        for h in range(Hkv):
            idx = np.asarray(slots[b, h], np.int64)
            ti = torch.from_numpy(idx).to(DEV)
            assert torch.equal(gk[b, h].index_select(0, ti), dev(st.K[b, h, idx], dt)) and \
                torch.equal(gv[b, h].index_select(0, ti), dev(st.V[b, h, idx], dt)), \
                f"{where} cache rows ({b},{h})"


def compare_step(g: dict, r: dict, st_after: oracle.H2OState, n_before: int, pos_before,
                 P: int, W: int, dtype: str, where: str = "", rows: str = "all") -> int:
    compare_attention(g, r, n_before, dtype, where)
    tol = TOL[dtype]
    e = rel_err(g["phi_updated"][:, :, :n_before], r["phi_updated"][:, :, :n_before])
    assert e.max(initial=0.0) <= tol["cs_rel"], f"{where} phi_updated rel {e.max():.3e}"
    swaps = compare_victims(g["freed_slots"], r["freed_slots"], r["rank"], pos_before,
                            n_before, P, W, where)
    if swaps == 0:
        assert (g["freed_slots"] == r["freed_slots"]).all(), f"{where} freed slots"
        assert (g["pos"] == st_after.pos).all(), f"{where} pos after insert"
        dt = TORCH_DT[dtype]
        if rows == "all":
            assert torch.equal(g["K"], dev(st_after.K, dt)) and \
                torch.equal(g["V"], dev(st_after.V, dt)), f"{where} cache rows after insert"
        else:                       # the rows this step wrote
            compare_rows(g["K"], g["V"], st_after, g["freed_slots"], dtype, where)
        n = st_after.n
        e = rel_err(g["phi"][:, :, :n], st_after.phi[:, :, :n]).max()
        assert e <= tol["cs_rel"], f"{where} phi after insert rel {e:.3e}"
        assert g["n"] == st_after.n
    return swaps


def run_chain(wl, chunks, get_inputs, cache=None, st=None, resync="on_divergence",
              score_mode="h2o", layer=0, rows="all"):
    """Drive GPU and oracle over the given chunks; return the number of near-tie swaps.

    resync: "on_divergence" reloads the GPU state from the oracle only after an
    accepted near-tie swap (free-running); "scores" also loads the oracle's scores
    (rounded to float32) after every chunk, so score rounding does not accumulate
    (teacher forcing: the K / V rows and positions are already bit-identical when the
    victims matched); "always" reloads the whole state after every chunk.
    rows: "all" compares every cache row after every chunk; "freed" only the rows
    the chunk wrote (and the whole cache once after the last chunk)."""
    dims = dims_of(wl)
    cache = cache or h2o.H2OCache(dims, DEV)
    st = st or oracle.H2OState.empty(wl.batch, wl.n_kv_heads, wl.capacity, wl.head_dim)
    swaps = 0
    for c in chunks:
        x = get_inputs(c)
        n_before, pos_before, P = st.n, st.pos.copy(), st.P
        assert cache.n_valid == st.n and cache.next_pos == st.P
        g = gpu_chunk(cache, x, wl.sm_scale, wl.dtype, score_mode)
        r = oracle.h2o_step(st, x["q"], x["k"], x["v"], wl.sm_scale, wl.recent_window,
                            score_mode)
        s = compare_step(g, r, st, n_before, pos_before, P, wl.recent_window, wl.dtype,
                         where=f"chunk {c}:", rows=rows)
        swaps += s
        if resync == "always" or s:
            load_oracle_state(cache, st, wl.dtype)
        elif resync == "scores":
            cache.score.copy_(dev(st.phi.astype(np.float32), torch.float32))
    if rows != "all":
        dt = TORCH_DT[wl.dtype]
        assert torch.equal(cache.k, dev(st.K, dt)) and torch.equal(cache.v, dev(st.V, dt)), \
            "cache rows after the last chunk"
        assert (host(cache.pos) == st.pos).all(), "positions after the last chunk"
    return swaps
