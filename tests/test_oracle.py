"""The oracle against its pins, and planted mistakes against the pins (CPU only)."""
import importlib.util
import os
import sys
import types

import pytest

import oracle
import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "h2o_oracle.py")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


# Each entry plants one plausible mistake in a copy of the oracle's source; at least one
# pin must fail on it.  (old text, new text, description)
MUTANTS = [
    ("(t[None, :] <= q_pos[:, None])", "(t[None, :] < q_pos[:, None])", "diagonal masked"),
    ("(t[None, :] >= 0) & ", "", "empty-slot marker visible"),
    ("np.lexsort((eligible, score[b, g, eligible]))",
     "np.lexsort((-eligible, score[b, g, eligible]))", "ties to the highest slot"),
    ("state.pos[b, g, :n] < P - W", "state.pos[b, g, :n] <= P - W", "window off by one"),
    ("summed += m.sum(axis=0)", "summed += m.sum(axis=0) / G", "group averaged, not summed"),
    ("state.phi[b, g, j] = colsum_new[b, g, i]", "state.phi[b, g, j] = 0.0",
     "new tokens start at score 0"),
    ("s = sm_scale * (q[b, h] @ keys.T)", "s = sm_scale * (q[b, h] @ keys.T) * sm_scale",
     "scale applied twice"),
    ("out[b, h] = m @ values", "out[b, h] = m.T[:S].T @ values[:S] if False else m @ keys",
     "keys used as values"),
    ("lse[b, h] = row_max[:, 0] + np.log(row_sum[:, 0])", "lse[b, h] = np.log(row_sum[:, 0])",
     "lse without the row max"),
    ("row_max = s.max(axis=1, keepdims=True)", "row_max = np.zeros_like(s[:, :1])",
     "softmax without its max subtraction"),
    ("victims[b, g] = np.sort(eligible[order[:k]])", "victims[b, g] = np.sort(eligible[order[-k:]])",
     "largest scores evicted"),
    ("np.arange(state.n, n_new)", "np.arange(state.n + 1, n_new + 1)", "empty slots off by one"),
    ("state.pos[b, g, j] = state.P + i", "state.pos[b, g, j] = state.P + i + 1",
     "inserted position off by one"),
    ("t_now = state.P + S", "t_now = state.P", "h2o-norm age off by S"),
    ("return state.phi / (t_now - state.pos).astype(np.float64)",
     "return state.phi / (t_now - state.pos + 1).astype(np.float64)", "h2o-norm age plus one"),
    ("state.pos[b, g, :n] >= beta", "state.pos[b, g, :n] > beta", "lastrec sink off by one"),
    ("np.sort(eligible[oldest[:k]])", "np.sort(eligible[oldest[-k:]])", "lastrec evicts newest"),
    ("    update_scores(state, colsum)\n", "    update_scores(state, colsum * 0.5)\n",
     "buffer form halves the scores"),
    ("np.asarray(v_new, np.float64), np.zeros((B, Hkv, S)))",
     "np.asarray(v_new, np.float64), np.ones((B, Hkv, S)))", "buffer form new score not zero"),
    ("            keys, values, t = state.K[b, g, :n], state.V[b, g, :n], state.pos[b, g, :n]",
     "            keys, values, t = state.K[b, g, :n], state.V[b, g, :n], state.pos[b, g, :n] - 1",
     "buffer mask off by one"),
    ("ds = m * (dm - (dout[b, h] * o).sum(axis=1, keepdims=True))", "ds = m * dm",
     "backward without the row term"),
    ("dkeys += sm_scale * (ds.T @ q[b, h])", "dkeys += ds.T @ q[b, h]", "backward dK unscaled"),
    ("dvalues += m.T @ dout[b, h]", "dvalues += 0.5 * (m.T @ dout[b, h])", "backward dV halved"),
    ("dq[b, h] = sm_scale * (ds @ keys)", "dq[b, h] = ds @ keys", "backward dQ unscaled"),
    ("h = g * G + hh", "h = hh * Hkv + g", "query heads interleaved over the KV heads"),
    ("return max(0, n + S - NC)", "return max(0, n + S - NC + 1)", "one eviction too many"),
]


def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert old in src, old
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    sys.modules["oracle_mutant"] = mod
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new,why", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_planted_mistakes_are_caught(old, new, why):
    mod = _mutant(old, new)
    failures = 0
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:        # AssertionError, or a crash caused by the mistake
            failures += 1
    assert failures > 0, f"no pin catches: {why}"
