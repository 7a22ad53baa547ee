"""Plain fp64 statement of one H2O chunk step (attention, scores, eviction, insert).

Test infrastructure only (see the package docstring).  Notation follows the
montaan paper page of "Learning how to Forget: Fine-tuning for Long-Context
Sparse Attention":

* ``N_C`` cache slots per (sequence b, KV head), chunk length ``S``;
* ``t(b,h,j)`` the token position held in slot j ("Improvements to H2O",
  item 2), stored here as ``pos[b, g, j]`` with -1 for an empty slot;
* ``m_{b,h,i,j}`` the attention weight of query row i on key j, and the summed
  weights ``sum_i m_{b,h,i,j}`` that the fast kernels should return
  ("Kernel Support Needs");
* ``phi_h2o(b,h,j)`` the H2O score: accumulated summed weights; new content
  overwrites the slots with the smallest score ("Improvements to H2O",
  item 2), optionally normalised by age (``h2o-norm``).

Readings taken where the pages are silent or garbled:

* query row i of a chunk starting at position P sits at position P+i; key j is
  visible to it iff 0 <= t(j) <= P+i (the implicit causal mask of "Kernel
  Support Needs", with the empty-slot marker -1 never visible);
* the chunk attends to the valid cache slots and to its own keys, and only
  then are scores accumulated, victims chosen and the chunk inserted;
* the score of a KV head sums the summed weights of all query heads sharing
  it (GQA group), over every query row of the chunk;
* eviction count k = max(0, n + S - N_C); eligible slots are the filled ones
  whose position is older than P - W; victims are the k smallest by
  (score, slot index); chunk token i goes to the i-th smallest freed slot;
* a newly inserted token starts with its own in-chunk summed weight as score;
* h2o-norm divides the score by the age t - t(j) with t = P + S;
* lastrec ("Experimental Validation", the lr policy: the first beta and the
  last N_C - beta tokens stay) evicts the k oldest filled slots whose position
  is at least beta, and refuses a chunk when fewer are eligible;
* the insert-first buffer form (the positional mask of "Kernel Support Needs"
  over the fixed-size buffer) chooses the victims on the scores before the
  chunk, writes the chunk with score 0, then attends over the N_C slots; the
  new tokens' scores are then their own summed weights, as in the other order;
* the backward ("Gradient Computation Strategy", item 1: the policy's choices
  are replayed, not differentiated) is that of masked softmax attention over
  the chunk's fixed keys and mask.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class H2OState:
    """One layer's cache: arrays shaped (B, Hkv, N_C[, d]); ``n`` filled slots; next position ``P``."""
    K: np.ndarray
    V: np.ndarray
    pos: np.ndarray
    phi: np.ndarray
    n: int = 0
    P: int = 0
    log: list = field(default_factory=list)   # per step: freed slots (B, Hkv, S)

    @classmethod
    def empty(cls, B, Hkv, NC, d):
        return cls(K=np.zeros((B, Hkv, NC, d)), V=np.zeros((B, Hkv, NC, d)),
                   pos=np.full((B, Hkv, NC), -1, np.int64), phi=np.zeros((B, Hkv, NC)))

    @classmethod
    def from_arrays(cls, k, v, pos, phi, n, P):
        return cls(K=np.asarray(k, np.float64).copy(), V=np.asarray(v, np.float64).copy(),
                   pos=np.asarray(pos, np.int64).copy(), phi=np.asarray(phi, np.float64).copy(),
                   n=int(n), P=int(P))

    def copy(self):
        return H2OState(self.K.copy(), self.V.copy(), self.pos.copy(), self.phi.copy(),
                        self.n, self.P, list(self.log))

    @property
    def capacity(self):
        return self.K.shape[2]


def attend_chunk(state: H2OState, q, k_new, v_new, sm_scale: float):
    """Chunk attention with the summed attention weights.

    q: (B, Hq, S, d); k_new, v_new: (B, Hkv, S, d).  Keys are the n filled
    slots followed by the chunk's own S keys (position P+i').  Query head h
    reads KV head h // G.

    Returns O (B,Hq,S,d), lse (B,Hq,S) natural log, colsum_cache (B,Hkv,N_C)
    (zero beyond n) and colsum_new (B,Hkv,S): sum over the chunk's query rows
    and the G query heads of each KV head of the softmax weights m_{b,h,i,j}.
    """
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    B, Hq, S, d = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    n, P, NC = state.n, state.P, state.capacity
    out = np.zeros((B, Hq, S, d))
    lse = np.zeros((B, Hq, S))
    colsum_cache = np.zeros((B, Hkv, NC))
    colsum_new = np.zeros((B, Hkv, S))
    q_pos = P + np.arange(S)
    for b in range(B):
        for g in range(Hkv):
            keys = np.concatenate([state.K[b, g, :n], k_new[b, g]])
            values = np.concatenate([state.V[b, g, :n], v_new[b, g]])
            t = np.concatenate([state.pos[b, g, :n], q_pos])       # t(b,g,j)
            visible = (t[None, :] >= 0) & (t[None, :] <= q_pos[:, None])
            summed = np.zeros(n + S)
            for hh in range(G):
                h = g * G + hh
                s = sm_scale * (q[b, h] @ keys.T)                      # (S, n+S)
                s = np.where(visible, s, -np.inf)
                row_max = s.max(axis=1, keepdims=True)
                e = np.exp(s - row_max)
                row_sum = e.sum(axis=1, keepdims=True)
                m = e / row_sum                                         # m_{b,h,i,j}
                out[b, h] = m @ values
                lse[b, h] = row_max[:, 0] + np.log(row_sum[:, 0])
                summed += m.sum(axis=0)                                 # sum_i m_{b,h,i,j}
            colsum_cache[b, g, :n] = summed[:n]
            colsum_new[b, g] = summed[n:]
    return out, lse, colsum_cache, colsum_new


def update_scores(state: H2OState, colsum_cache) -> None:
    """phi_h2o(b,g,j) += summed weights of this chunk, for the filled slots j < n."""
    n = state.n
    state.phi[:, :, :n] += np.asarray(colsum_cache, np.float64)[:, :, :n]


def eviction_count(n: int, S: int, NC: int) -> int:
    return max(0, n + S - NC)


def selection_scores(state: H2OState, S: int, score_mode: str = "h2o"):
    """Per-slot value the victims are ranked by: phi (h2o) or phi / (t - t(j)) (h2o-norm)."""
    if score_mode == "h2o":
        return state.phi
    if score_mode == "h2o_norm":
        # phi / (t - t(j)) with t = P + S: the age counts the chunk being processed,
        # so it is at least 1 for every cached token.
        t_now = state.P + S
        return state.phi / (t_now - state.pos).astype(np.float64)
    raise ValueError(score_mode)


def select_victims(state: H2OState, S: int, W: int, score_mode: str = "h2o"):
    """Victim slots per (b, g), ascending slot index: shape (B, Hkv, k).

    Eligible: filled slots j < n with t(j) < P - W.  The k = n + S - N_C slots
    with the smallest (score, slot index) are evicted; a full sort does it.
    """
    B, Hkv, NC = state.pos.shape
    n, P = state.n, state.P
    k = eviction_count(n, S, NC)
    victims = np.zeros((B, Hkv, k), np.int64)
    if k == 0:
        return victims
    score = selection_scores(state, S, score_mode)
    for b in range(B):
        for g in range(Hkv):
            slots = np.arange(n)
            eligible = slots[state.pos[b, g, :n] < P - W]
            if eligible.size < k:
                raise ValueError(f"cannot evict {k} slots: only {eligible.size} eligible")
            order = np.lexsort((eligible, score[b, g, eligible]))   # by score, then slot
            victims[b, g] = np.sort(eligible[order[:k]])
    return victims


def evict_and_insert(state: H2OState, victims, k_new, v_new, colsum_new):
    """Write the chunk into the freed slots; return freed_slots (B, Hkv, S).

    Targets are the victims together with the empty slots [n, min(N_C, n+S)),
    ascending; chunk token i goes to the i-th target with t = P+i and its own
    in-chunk summed weight as initial score.  Then n and P advance.
    """
    B, Hkv, S, _ = np.shape(k_new)
    NC = state.capacity
    n_new = min(NC, state.n + S)
    freed = np.zeros((B, Hkv, S), np.int64)
    for b in range(B):
        for g in range(Hkv):
            targets = np.sort(np.concatenate([victims[b, g], np.arange(state.n, n_new)]))
            assert targets.size == S
            for i, j in enumerate(targets):
                state.K[b, g, j] = k_new[b, g, i]
                state.V[b, g, j] = v_new[b, g, i]
                state.pos[b, g, j] = state.P + i
                state.phi[b, g, j] = colsum_new[b, g, i]
            freed[b, g] = targets
    state.n = n_new
    state.P += S
    state.log.append(freed)
    return freed


def h2o_step(state: H2OState, q, k_new, v_new, sm_scale: float, W: int,
             score_mode: str = "h2o"):
    """One chunk: attend, accumulate scores, select victims, insert.  Mutates ``state``."""
    S = np.shape(q)[2]
    out, lse, cs_cache, cs_new = attend_chunk(state, q, k_new, v_new, sm_scale)
    update_scores(state, cs_cache)
    phi_after_update = state.phi.copy()
    rank = selection_scores(state, S, score_mode).copy()
    victims = select_victims(state, S, W, score_mode)
    evicted_phi = np.take_along_axis(state.phi, victims, axis=2) if victims.size else \
        np.zeros(victims.shape)
    freed = evict_and_insert(state, victims, np.asarray(k_new, np.float64),
                             np.asarray(v_new, np.float64), cs_new)
    return {"out": out, "lse": lse, "colsum_cache": cs_cache, "colsum_new": cs_new,
            "phi_updated": phi_after_update, "rank": rank, "victims": victims,
            "evicted_phi": evicted_phi, "freed_slots": freed}


# --------------------------------------------------------------------- lastrec
def select_victims_lastrec(state: H2OState, S: int, beta: int):
    """Victim slots of the lastrec policy, ascending slot index: shape (B, Hkv, k).

    lastrec keeps the first beta tokens and the last N_C - beta tokens of the
    sequence (montaan paper page, "Experimental Validation", the lr policy).
    When the chunk does not fit, the k = n + S - N_C oldest filled slots among
    those at position >= beta are evicted (positions are unique: no ties).
    """
    B, Hkv, NC = state.pos.shape
    n = state.n
    k = eviction_count(n, S, NC)
    victims = np.zeros((B, Hkv, k), np.int64)
    if k == 0:
        return victims
    for b in range(B):
        for g in range(Hkv):
            slots = np.arange(n)
            eligible = slots[state.pos[b, g, :n] >= beta]
            if eligible.size < k:
                raise ValueError(f"cannot evict {k} slots: only {eligible.size} eligible")
            oldest = np.argsort(state.pos[b, g, eligible], kind="stable")
            victims[b, g] = np.sort(eligible[oldest[:k]])
    return victims


def lastrec_step(state: H2OState, q, k_new, v_new, sm_scale: float, beta: int):
    """One chunk under lastrec: attend (the summed weights are not needed by the
    policy), evict by position, insert with score 0.  Mutates ``state``."""
    S = np.shape(q)[2]
    out, lse, _, cs_new = attend_chunk(state, q, k_new, v_new, sm_scale)
    victims = select_victims_lastrec(state, S, beta)
    freed = evict_and_insert(state, victims, np.asarray(k_new, np.float64),
                             np.asarray(v_new, np.float64), np.zeros(np.shape(cs_new)))
    return {"out": out, "lse": lse, "victims": victims, "freed_slots": freed}


# ------------------------------------------------------------ insert-first buffer form
def attend_buffer(state: H2OState, q, P: int, sm_scale: float):
    """Chunk attention over the slot buffer alone, the chunk already written into it.

    Query row i sits at position P + i and sees slot j iff 0 <= t(j) <= P + i
    (the positional mask over the fixed-size buffer, "Kernel Support Needs").
    Returns O, lse and the summed weights per slot (B, Hkv, N_C), zero beyond n.
    """
    q = np.asarray(q, np.float64)
    B, Hq, S, d = q.shape
    Hkv = state.K.shape[1]
    G = Hq // Hkv
    n, NC = state.n, state.capacity
    out = np.zeros((B, Hq, S, d))
    lse = np.zeros((B, Hq, S))
    colsum = np.zeros((B, Hkv, NC))
    q_pos = P + np.arange(S)
    for b in range(B):
        for g in range(Hkv):
            keys, values, t = state.K[b, g, :n], state.V[b, g, :n], state.pos[b, g, :n]
            visible = (t[None, :] >= 0) & (t[None, :] <= q_pos[:, None])
            for hh in range(G):
                h = g * G + hh
                s = np.where(visible, sm_scale * (q[b, h] @ keys.T), -np.inf)
                row_max = s.max(axis=1, keepdims=True)
                e = np.exp(s - row_max)
                row_sum = e.sum(axis=1, keepdims=True)
                m = e / row_sum
                out[b, h] = m @ values
                lse[b, h] = row_max[:, 0] + np.log(row_sum[:, 0])
                colsum[b, g, :n] += m.sum(axis=0)
    return out, lse, colsum


def buffer_step(state: H2OState, q, k_new, v_new, sm_scale: float, W: int,
                score_mode: str = "h2o"):
    """One chunk in the insert-first buffer form: the victims are chosen on the
    scores before the chunk, the chunk is written into the targets with score 0,
    the chunk attends over the N_C-slot buffer under the positional mask, and
    every filled slot's score accumulates its summed weight.  Mutates ``state``."""
    B, Hkv, S, _ = np.shape(k_new)
    P = state.P
    victims = select_victims(state, S, W, score_mode)
    evicted_phi = np.take_along_axis(state.phi, victims, axis=2) if victims.size else \
        np.zeros(victims.shape)
    freed = evict_and_insert(state, victims, np.asarray(k_new, np.float64),
                             np.asarray(v_new, np.float64), np.zeros((B, Hkv, S)))
    out, lse, colsum = attend_buffer(state, q, P, sm_scale)
    update_scores(state, colsum)
    return {"out": out, "lse": lse, "colsum": colsum, "victims": victims,
            "evicted_phi": evicted_phi, "freed_slots": freed}


# ------------------------------------------------------------------- backward
def attend_chunk_backward(state: H2OState, q, k_new, v_new, dout, sm_scale: float,
                          excluded=None):
    """Gradients of the chunk attention's output with the cache decisions fixed.

    The policy's choices are replayed rather than differentiated (montaan paper
    page, "Gradient Computation Strategy", item 1), so the keys and the mask of
    ``attend_chunk`` are constants here and the gradient is that of masked
    softmax attention.  ``excluded`` (B, Hkv, N_C) bool marks cache slots that
    are not keys (the buffer form's overwritten slots).

    Per query head, with m = softmax(s) over the visible keys and dm = dO V^T:
        dV += m^T dO,  ds = m * (dm - rowsum(dO * O)),
        dQ = sm_scale * ds K,  dK += sm_scale * ds^T Q.
    Returns dq (B,Hq,S,d), dk_new, dv_new (B,Hkv,S,d) and dk_cache, dv_cache
    (B,Hkv,N_C,d), zero beyond n and at excluded slots.
    """
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    dout = np.asarray(dout, np.float64)
    B, Hq, S, d = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    n, P, NC = state.n, state.P, state.capacity
    dq = np.zeros((B, Hq, S, d))
    dk_new = np.zeros((B, Hkv, S, d))
    dv_new = np.zeros((B, Hkv, S, d))
    dk_cache = np.zeros((B, Hkv, NC, d))
    dv_cache = np.zeros((B, Hkv, NC, d))
    q_pos = P + np.arange(S)
    for b in range(B):
        for g in range(Hkv):
            keys = np.concatenate([state.K[b, g, :n], k_new[b, g]])
            values = np.concatenate([state.V[b, g, :n], v_new[b, g]])
            t = np.concatenate([state.pos[b, g, :n], q_pos])
            visible = (t[None, :] >= 0) & (t[None, :] <= q_pos[:, None])
            if excluded is not None:
                visible[:, :n] &= ~np.asarray(excluded[b, g, :n], bool)[None, :]
            dkeys = np.zeros_like(keys)
            dvalues = np.zeros_like(values)
            for hh in range(G):
                h = g * G + hh
                s = np.where(visible, sm_scale * (q[b, h] @ keys.T), -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                m = e / e.sum(axis=1, keepdims=True)
                o = m @ values
                dm = dout[b, h] @ values.T
                ds = m * (dm - (dout[b, h] * o).sum(axis=1, keepdims=True))
                dvalues += m.T @ dout[b, h]
                dq[b, h] = sm_scale * (ds @ keys)
                dkeys += sm_scale * (ds.T @ q[b, h])
            dk_cache[b, g, :n], dk_new[b, g] = dkeys[:n], dkeys[n:]
            dv_cache[b, g, :n], dv_new[b, g] = dvalues[:n], dvalues[n:]
    return dq, dk_new, dv_new, dk_cache, dv_cache

