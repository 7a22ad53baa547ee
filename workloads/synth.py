"""Seeded synthetic inputs for the H2O chunked sparse-attention workloads.

The pages ("Learning how to Forget: Fine-tuning for Long-Context Sparse
Attention", montaan paper page and metallab summary) evaluate on Helmet
long-context datasets with a Qwen3-4B checkpoint.  Neither is available here,
so these generators stand in for them with random tensors of the same
attention shape (32 query heads, 8 KV heads, head_dim 128) at the context
lengths the pages quote (64k / 128k tokens) and the chunk sizes of their
Tables 1 and 5 (1024 / 2048).

Every draw comes from ``numpy.random.PCG64`` seeded with
``SeedSequence([workload key, layer, stream, index])`` so that any chunk (or
decode step) can be generated on its own, on any machine, bit for bit.
Values are drawn in float32 and, for bf16 workloads, rounded to bf16 with
round-to-nearest-even; both the oracle and the GPU consume those exact bits.

Nothing here computes attention, scores or evictions.
"""
from __future__ import annotations

from dataclasses import dataclass
from functools import lru_cache

import numpy as np

_STREAMS = {"q": 1, "k": 2, "v": 3, "heavy": 4, "norm": 5, "state": 6, "phi": 7}


@dataclass(frozen=True)
class Workload:
    key: int                 # workload id mixed into every seed
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    capacity: int            # N_C: cache slots per (sequence, KV head)
    recent_window: int       # W: most recent cached positions protected from eviction
    chunk: int               # S: query tokens per chunk (1 for decode)
    seq_len: int             # tokens processed per layer (prefill) / steps (decode)
    dtype: str               # "f32" or "bf16": storage and MFMA input type
    sm_scale: float          # softmax scale applied to q.k
    layers: int = 1
    key_scale: float = 1.0   # multiplies every drawn key
    heavy_kind: str = "shared_dir"   # "shared_dir" | "query_mean"
    heavy_count: int = 0     # boosted positions (per sequence)
    heavy_alpha: float = 0.0  # boost length along the heavy direction
    key_norm_sigma: float = 0.0   # per-(layer, KV head) LogNormal(0, sigma) key multiplier
    decode: bool = False     # True: S = 1 steps after a full initial cache

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk

    @property
    def total_positions(self) -> int:
        """Positions that exist in the sequence (decode: initial cache + steps)."""
        return self.capacity + self.seq_len if self.decode else self.seq_len


WORKLOADS = {
    1: Workload(1, "plumbing_f32_d64", batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64,
                capacity=256, recent_window=32, chunk=64, seq_len=1024, dtype="f32",
                sm_scale=1.0, key_scale=1.0 / 8.0, heavy_kind="query_mean",
                heavy_count=8, heavy_alpha=3.0),
    2: Workload(2, "qwen3_4b_chunk1k_ctx64k", batch=1, n_q_heads=32, n_kv_heads=8,
                head_dim=128, capacity=8192, recent_window=256, chunk=1024, seq_len=65536,
                dtype="bf16", sm_scale=128 ** -0.5, heavy_kind="shared_dir",
                heavy_count=655, heavy_alpha=2.0),
    3: Workload(3, "qwen3_4b_chunk2k_ctx128k", batch=1, n_q_heads=32, n_kv_heads=8,
                head_dim=128, capacity=16384, recent_window=512, chunk=2048,
                seq_len=131072, dtype="bf16", sm_scale=128 ** -0.5,
                heavy_kind="shared_dir", heavy_count=1311, heavy_alpha=2.0,
                key_norm_sigma=0.5),
    4: Workload(4, "qwen3_4b_36layer_chunk1k_ctx128k", batch=1, n_q_heads=32, n_kv_heads=8,
                head_dim=128, capacity=8192, recent_window=256, chunk=1024, seq_len=131072,
                dtype="bf16", sm_scale=128 ** -0.5, layers=36, heavy_kind="shared_dir",
                heavy_count=1311, heavy_alpha=2.0),
    5: Workload(5, "decode_b16_cache16k", batch=16, n_q_heads=32, n_kv_heads=8,
                head_dim=128, capacity=16384, recent_window=512, chunk=1, seq_len=512,
                dtype="bf16", sm_scale=128 ** -0.5, heavy_kind="query_mean",
                heavy_count=8, heavy_alpha=3.0, decode=True),
}


def workload(key: int, **overrides) -> Workload:
    """A registered workload, optionally with fields replaced (smaller test shapes)."""
    wl = WORKLOADS[key]
    if overrides:
        fields = dict(wl.__dict__)
        fields.update(overrides)
        wl = Workload(**fields)
    return wl


def rng_for(wl: Workload, layer: int, stream: str, index: int) -> np.random.Generator:
    seq = np.random.SeedSequence([wl.key, layer, _STREAMS[stream], index])
    return np.random.Generator(np.random.PCG64(seq))


# --------------------------------------------------------------------------- bf16
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values exactly representable in bf16 (nearest, ties to even)."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def _store(wl: Workload, x: np.ndarray) -> np.ndarray:
    return bf16_round(x) if wl.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


# ------------------------------------------------------------------- heavy hitters
def _draw_q(wl: Workload, layer: int, index: int, n_tok: int) -> np.ndarray:
    r = rng_for(wl, layer, "q", index)
    return _store(wl, r.standard_normal((wl.batch, wl.n_q_heads, n_tok, wl.head_dim),
                                        dtype=np.float32))


@lru_cache(maxsize=16)
def heavy_boost(wl: Workload, layer: int):
    """Boosted positions (batch, count) and unit directions (batch, head_dim).

    ``shared_dir``: one seeded unit vector and one position set for every
    sequence and KV head.  ``query_mean``: per sequence, the normalised mean of
    all of that sequence's query vectors (over tokens and heads), and a seeded
    position set per sequence.
    """
    r = rng_for(wl, layer, "heavy", 0)
    n_pos = wl.total_positions
    if wl.heavy_count == 0:
        return (np.zeros((wl.batch, 0), np.int64),
                np.zeros((wl.batch, wl.head_dim), np.float32))
    if wl.heavy_kind == "shared_dir":
        pos = np.sort(r.choice(n_pos, wl.heavy_count, replace=False)).astype(np.int64)
        u = r.standard_normal(wl.head_dim).astype(np.float64)
        u /= np.linalg.norm(u)
        return (np.broadcast_to(pos, (wl.batch, wl.heavy_count)).copy(),
                np.broadcast_to(u.astype(np.float32), (wl.batch, wl.head_dim)).copy())
    if wl.heavy_kind == "query_mean":
        pos = np.stack([np.sort(r.choice(n_pos, wl.heavy_count, replace=False))
                        for _ in range(wl.batch)]).astype(np.int64)
        acc = np.zeros((wl.batch, wl.head_dim), np.float64)
        count = 0
        if wl.decode:
            for t in range(wl.seq_len):
                q = _draw_q(wl, layer, t, 1)
                acc += q.astype(np.float64).sum(axis=(1, 2))
                count += q.shape[1] * q.shape[2]
        else:
            for c in range(wl.n_chunks):
                q = _draw_q(wl, layer, c, wl.chunk)
                acc += q.astype(np.float64).sum(axis=(1, 2))
                count += q.shape[1] * q.shape[2]
        u = acc / count
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        return pos, u.astype(np.float32)
    raise ValueError(wl.heavy_kind)


@lru_cache(maxsize=16)
def _key_norms(wl: Workload, layer: int) -> np.ndarray:
    if wl.key_norm_sigma == 0.0:
        return np.ones(wl.n_kv_heads, np.float32)
    r = rng_for(wl, layer, "norm", 0)
    return r.lognormal(0.0, wl.key_norm_sigma, wl.n_kv_heads).astype(np.float32)


def _make_keys(wl: Workload, layer: int, raw: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """raw: (B, Hkv, T, d) float32 normals; positions: (B, Hkv, T) token positions."""
    k = raw * np.float32(wl.key_scale)
    hpos, hdir = heavy_boost(wl, layer)
    if hpos.shape[1]:
        for b in range(wl.batch):
            hit = np.isin(positions[b], hpos[b])          # (Hkv, T)
            k[b][hit] += np.float32(wl.heavy_alpha) * hdir[b]
    k *= _key_norms(wl, layer)[None, :, None, None]
    return _store(wl, k)


# ---------------------------------------------------------------------- prefill
def chunk_inputs(wl: Workload, layer: int, c: int) -> dict:
    """q (B,Hq,S,d), k and v (B,Hkv,S,d) for chunk c: positions c*S ... c*S+S-1."""
    S = wl.chunk
    q = _draw_q(wl, layer, c, S)
    kraw = rng_for(wl, layer, "k", c).standard_normal(
        (wl.batch, wl.n_kv_heads, S, wl.head_dim), dtype=np.float32)
    v = rng_for(wl, layer, "v", c).standard_normal(
        (wl.batch, wl.n_kv_heads, S, wl.head_dim), dtype=np.float32)
    pos = np.broadcast_to(c * S + np.arange(S), (wl.batch, wl.n_kv_heads, S))
    return {"q": q, "k": _make_keys(wl, layer, kraw, pos), "v": _store(wl, v),
            "start": c * S}


def steady_state(wl: Workload, layer: int, start: int, seed: int = 0,
                 tie_fraction: float = 0.05) -> dict:
    """A full cache as it could stand before the chunk at position ``start``.

    Per (sequence, KV head): the previous chunk's S positions plus a random
    subset of older positions, in random slot order; keys and values drawn
    fresh for each slot; scores positive LogNormal draws with a fraction of
    them set to a few shared values so that exact ties occur.
    """
    B, Hkv, NC, d, S = wl.batch, wl.n_kv_heads, wl.capacity, wl.head_dim, wl.chunk
    if start < NC:
        raise ValueError("steady_state needs start >= capacity")
    r = rng_for(wl, layer, "state", 1000 + seed)
    pos = np.empty((B, Hkv, NC), np.int64)
    recent = np.arange(start - S, start)
    for b in range(B):
        for g in range(Hkv):
            older = r.choice(start - S, NC - S, replace=False)
            pos[b, g] = r.permutation(np.concatenate([recent, older]))
    kraw = r.standard_normal((B, Hkv, NC, d), dtype=np.float32)
    v = r.standard_normal((B, Hkv, NC, d), dtype=np.float32)
    phi = (wl.group * r.lognormal(0.0, 1.0, (B, Hkv, NC))).astype(np.float32)
    n_tie = int(tie_fraction * NC)
    if n_tie:
        levels = np.sort(phi.reshape(-1))[[NC // 8, NC // 4, NC // 2]].astype(np.float32)
        for b in range(B):
            for g in range(Hkv):
                idx = r.choice(NC, n_tie, replace=False)
                phi[b, g, idx] = levels[r.integers(0, 3, n_tie)]
    return {"k": _make_keys(wl, layer, kraw, pos), "v": _store(wl, v),
            "pos": pos.astype(np.int32), "phi": phi, "n": NC, "start": start}


# ----------------------------------------------------------------------- decode
def decode_initial_state(wl: Workload, layer: int = 0, batches=None) -> dict:
    """Full cache for the decode workload: slot j holds position j (0 <= j < N_C).

    Scores are a stand-in for what a causal prefill would have left: the
    column sum of uniform causal attention over N_C tokens (G times the tail of
    the harmonic series) times LogNormal(0, 0.25) jitter.
    """
    assert wl.decode
    bs = range(wl.batch) if batches is None else batches
    NC, Hkv, d, G = wl.capacity, wl.n_kv_heads, wl.head_dim, wl.group
    ks, vs, phis = [], [], []
    tail = np.cumsum((1.0 / np.arange(1, NC + 1, dtype=np.float64))[::-1])[::-1]
    hpos, hdir = heavy_boost(wl, layer)
    for b in bs:
        r = rng_for(wl, layer, "state", b)
        kraw = r.standard_normal((Hkv, NC, d), dtype=np.float32) * np.float32(wl.key_scale)
        hit = hpos[b][hpos[b] < NC]
        kraw[:, hit, :] += np.float32(wl.heavy_alpha) * hdir[b]
        kraw *= _key_norms(wl, layer)[:, None, None]
        ks.append(_store(wl, kraw))
        vs.append(_store(wl, r.standard_normal((Hkv, NC, d), dtype=np.float32)))
        jitter = r.lognormal(0.0, 0.25, (Hkv, NC))
        phis.append((G * tail[None, :] * jitter).astype(np.float32))
    nb = len(list(bs))
    pos = np.broadcast_to(np.arange(NC, dtype=np.int32), (nb, Hkv, NC)).copy()
    return {"k": np.stack(ks), "v": np.stack(vs), "pos": pos, "phi": np.stack(phis),
            "n": NC, "start": NC}


def decode_step_inputs(wl: Workload, t: int, layer: int = 0) -> dict:
    """q (B,Hq,1,d), k and v (B,Hkv,1,d) for decode step t at position N_C + t."""
    assert wl.decode
    q = _draw_q(wl, layer, t, 1)
    kraw = rng_for(wl, layer, "k", t).standard_normal(
        (wl.batch, wl.n_kv_heads, 1, wl.head_dim), dtype=np.float32)
    v = rng_for(wl, layer, "v", t).standard_normal(
        (wl.batch, wl.n_kv_heads, 1, wl.head_dim), dtype=np.float32)
    p = wl.capacity + t
    pos = np.full((wl.batch, wl.n_kv_heads, 1), p)
    return {"q": q, "k": _make_keys(wl, layer, kraw, pos), "v": _store(wl, v), "start": p}
