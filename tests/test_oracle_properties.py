"""Properties of the oracle over random tiny shapes (hypothesis): prompt
lengths that are not multiples of 64, head dims 4, 8 and 64, random budgets
and pool sizes, runs that cross block boundaries, data from a random layer
seed.  Each property is fixed by the pages or by the mathematics and is
checked here without the oracle's own routine for it:

* the selected sets are the union of two brute-force top-k's (numpy
  lexsort by score descending, block id ascending) over the candidates
  before the window (Eq. 7 read as U1);
* the query-agnostic part never takes back a block it dropped (the
  eviction rule), and the step-to-step overlap is at least ke / k;
* the pool: every selected block is resident after the step, in the slot
  phys names; the misses are exactly the selected blocks not resident
  before; free slots go first, lowest first; a miss never evicts a block of
  the step's set, and every evicted block was least recently used among the
  blocks outside the set;
* with every candidate selected the attention is dense causal softmax
  attention over [0, p], written out here in float64.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import nosa_inputs as NI
from oracle import nosa_oracle as O

SETTINGS = dict(max_examples=100, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _run(L, D, kq, ke, steps, layer, pool_slots=None, attend=False):
    w = NI.scaled(NI.WORKLOADS["tiny"], prompt_len=L, n_steps=steps, kq=kq, ke=ke, head_dim=D)
    K, V, lam = NI.unit_kv(w, 0, 0, layer=layer)
    q = NI.queries(w, layer=layer)[:, 0]
    tr = O.decode_unit(K, V, lam, q, w.positions(), kq, ke, bf16=False, pool_slots=pool_slots, attend=attend)
    return w, K, V, lam, q, tr


def _top(scores, n):
    """Indices of the n best scores, score descending then index ascending."""
    idx = np.arange(len(scores))
    order = np.lexsort((idx, -np.asarray(scores, dtype=np.float64)))
    return sorted(order[:n].tolist())


shapes = dict(
    L=st.integers(65, 2000).filter(lambda x: x % 64 != 0),
    D=st.sampled_from([4, 8, 64]),
    kq=st.integers(0, 6),
    ke=st.integers(0, 6),
    steps=st.integers(1, 140),
    layer=st.integers(0, 10_000),
)


@settings(**SETTINGS)
@given(**shapes)
def test_selection_is_the_union_of_two_brute_force_top_k(L, D, kq, ke, steps, layer):
    w, K, V, lam, q, tr = _run(L, D, kq, ke, steps, layer)
    E = O.block_eviction_scores(O.subblock_logit_means(lam))
    for t, p in enumerate(w.positions()):
        c = int(p) // 64
        g_q = _top(tr.s_q[t][:c], min(kq, c))
        g_e = _top(E[:c], min(ke, c))
        assert tr.gamma_q[t] == g_q and tr.gamma_e[t] == g_e
        assert tr.sel[t] == sorted(set(g_q) | set(g_e))
        assert all(0 <= j < c for j in tr.sel[t])


@settings(**SETTINGS)
@given(**shapes)
def test_eviction_rule_and_overlap_bound(L, D, kq, ke, steps, layer):
    w, K, V, lam, q, tr = _run(L, D, kq, ke, steps, layer)
    pos = w.positions()
    dropped = set()
    for t in range(len(tr.sel)):
        cur = set(tr.gamma_e[t])
        assert not (cur & dropped), t
        if t:
            dropped |= set(tr.gamma_e[t - 1]) - cur
            c = int(pos[t]) // 64
            S = tr.sel[t]
            if ke > 0 and c >= ke and S:
                held = set(tr.sel[t - 1]) | {int(pos[t - 1]) // 64}
                assert len(set(S) & held) / len(S) >= ke / (kq + ke) - 1e-12, t


@settings(**SETTINGS)
@given(extra=st.integers(1, 8), **shapes)
def test_pool_invariants(L, D, kq, ke, steps, layer, extra):
    k = kq + ke
    if k == 0:
        return
    P = k + extra
    w, K, V, lam, q, tr = _run(L, D, kq, ke, steps, layer, pool_slots=P)
    pos = w.positions()
    slot_block = [-1] * P
    last_use = [-1] * P
    for t, S in enumerate(tr.sel):
        c = int(pos[t]) // 64
        done = c - 1 if t and c > int(pos[t - 1]) // 64 else None
        ins = tr.insert_slot[t]
        if done is not None and done not in slot_block:
            # the completed block enters a free slot (the lowest), else a least
            # recently used one outside the set -- unless a miss takes it back
            free = [s for s in range(P) if slot_block[s] < 0]
            if free:
                target = free[0]
            else:
                cand = [s for s in range(P) if slot_block[s] not in S]
                target = min(cand, key=lambda s: (last_use[s], slot_block[s]))
            slot_block[target], last_use[target] = done, t - 1
            assert ins in (target, -1)
        else:
            assert ins == -1
        resident = {b for b in slot_block if b >= 0}
        misses = tr.misses[t]
        assert [b for b, _ in misses] == sorted(set(S) - resident)
        for b, s in misses:
            old = slot_block[s]
            if old >= 0:
                assert old not in S
                others = [x for x in range(P) if slot_block[x] >= 0 and slot_block[x] not in S and x != s]
                assert all((last_use[s], old) < (last_use[x], slot_block[x]) for x in others)
            else:
                assert s == min(x for x in range(P) if slot_block[x] < 0)
            slot_block[s] = b
        if ins >= 0:
            assert slot_block[ins] == done
        for b, s in zip(S, tr.phys[t]):
            assert slot_block[s] == b
            last_use[s] = t
        assert len({b for b in slot_block if b >= 0}) == sum(1 for b in slot_block if b >= 0) <= P


@settings(**SETTINGS)
@given(L=st.integers(65, 700).filter(lambda x: x % 64 != 0), D=st.sampled_from([4, 8, 64]),
       steps=st.integers(1, 6), layer=st.integers(0, 10_000))
def test_all_candidates_selected_is_dense_causal_attention(L, D, steps, layer):
    nb = (L + steps) // 64 + 1
    w, K, V, lam, q, tr = _run(L, D, nb, 0, steps, layer, attend=True)
    for t, p in enumerate(w.positions()):
        Kp, Vp = K[: p + 1].astype(np.float64), V[: p + 1].astype(np.float64)
        logits = q[t].astype(np.float64) @ Kp.T / np.sqrt(D)
        wts = np.exp(logits - logits.max(axis=1, keepdims=True))
        ref = (wts / wts.sum(axis=1, keepdims=True)) @ Vp
        assert np.allclose(tr.out[t], ref, rtol=0, atol=1e-5), t
