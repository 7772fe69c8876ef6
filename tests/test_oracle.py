"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a library routine, brute force, a closed
form, a stated invariant of the method, or a fixture worked by hand under
tests/golden/ (each fixture cites the passage it follows).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import nosa_oracle as O
import nosa_inputs as NI

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- rounding
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * 100
    # exact ties: low 16 bits = 0x8000, both parities of the kept part
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-38, 3e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.to_bf16(x), ref)


# ------------------------------------------------------------------ pooling
def test_pooling_order_fixture():
    g = _golden("pooling_small.json")["order_case"]
    K = np.array(g["tokens"], dtype=np.float32)[:, None]
    got = O.subblock_key_means(K, bf16=False)
    assert got.shape == (1, 1)
    assert got[0, 0] == np.float32(g["mean_f32"])
    # the logits follow the same fp32 order
    assert O.subblock_logit_means(K[:, 0])[0] == np.float32(g["mean_f32"])


def test_block_constant_keys_pool_to_the_key():
    rng = np.random.default_rng(1)
    for bf16 in (False, True):
        # 8 significant bits: every partial sum k*key (k <= 16) is exact in fp32
        keys = O.to_bf16(rng.standard_normal((7, 32)).astype(np.float32))
        K = np.repeat(keys, 64, axis=0)
        kbar = O.subblock_key_means(K, bf16)
        np.testing.assert_array_equal(kbar, np.repeat(keys, 4, axis=0))


def test_pooling_agrees_with_exact_sum_except_rounding_boundaries():
    rng = np.random.default_rng(2)
    K = O.to_bf16(rng.standard_normal((64 * 256, 128)).astype(np.float32))
    got = O.subblock_key_means(K, bf16=True)
    exact = K.astype(np.float64).reshape(-1, 16, 128).sum(axis=1) / 16.0
    alt = torch.from_numpy(exact).to(torch.bfloat16).to(torch.float32).numpy()
    diff = got != alt
    assert diff.mean() < 2e-3, diff.mean()
    # where they differ the two are adjacent bf16 values (one ulp apart)
    ulp = np.abs(got[diff].view(np.int32).astype(np.int64) - alt[diff].view(np.int32).astype(np.int64))
    assert np.all(ulp == (1 << 16))


def test_eviction_block_score_is_max_of_subblock_means():
    g = _golden("pooling_small.json")["eviction_case"]
    lam = np.repeat(np.array(g["subblock_values"], np.float32), 16)
    E = O.block_eviction_scores(O.subblock_logit_means(lam))
    assert E.shape == (1,) and E[0] == np.float32(g["E"])
    # block-constant logits give that constant
    vals = np.float32([0.25, -3.5, 7.0])
    E2 = O.block_eviction_scores(O.subblock_logit_means(np.repeat(vals, 64)))
    np.testing.assert_array_equal(E2, vals)


# ------------------------------------------------------------ query scores
def test_max_pool_of_scores_fixture():
    g = _golden("pooling_small.json")["maxpool_case"]
    keys = np.array(g["subblock_keys"], np.float32)
    K = np.repeat(keys, 16, axis=0)              # 64 tokens, constant per sub-block
    kbar = O.subblock_key_means(K, bf16=False)
    s = O.query_block_scores(np.array([g["q"]], np.float32), kbar, 1)
    assert s[0] == g["block_score"]


def test_query_scores_block_constant_closed_form():
    rng = np.random.default_rng(3)
    keys = rng.integers(-4, 5, size=(9, 16)).astype(np.float32)
    K = np.repeat(keys, 64, axis=0)
    kbar = O.subblock_key_means(K, bf16=False)
    q = rng.integers(-3, 4, size=(4, 16)).astype(np.float32)
    s = O.query_block_scores(q, kbar, 9)
    # integer data: the closed form is exact in any order
    expect = [float(sum(int(q[g, d]) * int(keys[b, d]) for g in range(4) for d in range(16)))
              for b in range(9)]
    assert list(s) == expect


def test_every_query_head_of_the_group_counts():
    # two orthogonal query heads; block 3 aligned with head 1, block 6 with head 0,
    # block 8 anti-aligned with both: the query-aware top-2 must be {3, 6} and
    # block 8 must rank last (reading U3: one selection from the whole group).
    rng = np.random.default_rng(4)
    D = 64
    q = np.zeros((2, D), np.float32)
    q[0, :32] = rng.standard_normal(32)
    q[1, 32:] = rng.standard_normal(32)
    keys = 0.05 * rng.standard_normal((10, D)).astype(np.float32)
    keys[3] = 3 * q[1] / np.linalg.norm(q[1])
    keys[6] = 3 * q[0] / np.linalg.norm(q[0])
    keys[8] = -3 * (q[0] + q[1]) / np.linalg.norm(q[0] + q[1])
    K = np.repeat(keys, 64, axis=0)
    s = O.query_block_scores(q, O.subblock_key_means(K, False), 10)
    assert sorted(O.top_blocks(s, 2)) == [3, 6]
    assert O.top_blocks(s, 10)[-1] == 8


def test_selection_invariant_to_positive_query_scale():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((64 * 40, 32)).astype(np.float32)
    kbar = O.subblock_key_means(K, False)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    a = O.top_blocks(O.query_block_scores(q, kbar, 40), 8)
    b = O.top_blocks(O.query_block_scores(q * np.float32(4.0), kbar, 40), 8)
    assert a == b


# -------------------------------------------------- chunk-shared selection (U20)
def _shared_case(seed, n_query=5, G=2, D=16, n_blk=12):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((64 * (n_blk + 1), D)).astype(np.float32)
    kbar = O.subblock_key_means(K, False)
    E = [float(v) for v in rng.standard_normal(n_blk + 1)]
    q = rng.standard_normal((n_query, G, D)).astype(np.float32)
    return kbar, E, q


def test_shared_selection_of_one_row_is_the_decode_selection():
    kbar, E, q = _shared_case(1, n_query=1)
    pos = 64 * 12 + 9
    want = O.select_blocks(O.query_block_scores(q[0], kbar, 12), E, 12, 3, 2)
    assert O.chunk_shared_selection(q, pos, kbar, E, 3, 2) == want


def test_shared_selection_brute_force():
    """Scores by explicit loops over rows, heads, dimensions and sub-blocks;
    the selected Gamma_q must out-rank every other candidate (ties by id)."""
    kbar, E, q = _shared_case(2)
    n_cand, kq, ke = 12, 4, 3
    gq, ge, S = O.chunk_shared_selection(q, 64 * n_cand + 30, kbar, E, kq, ke)
    score = []
    for j in range(n_cand):
        best = None
        for i in range(4):
            tot = 0.0
            for r in range(q.shape[0]):
                for g in range(q.shape[1]):
                    for d in range(q.shape[2]):
                        tot += float(q[r, g, d]) * float(kbar[4 * j + i, d])
            best = tot if best is None else max(best, tot)
        score.append(best)
    assert len(gq) == kq and len(ge) == ke
    for j in gq:
        for o in range(n_cand):
            if o not in gq:
                assert score[j] > score[o] + 1e-9 or (abs(score[j] - score[o]) <= 1e-9 and j < o)
    assert ge == sorted(O.top_blocks(E[:n_cand], ke))
    assert S == sorted(set(gq) | set(ge))


def test_shared_selection_ignores_row_order_and_duplication():
    kbar, E, q = _shared_case(3, n_query=6)
    pos = 64 * 12
    base = O.chunk_shared_selection(q, pos, kbar, E, 5, 2)
    assert O.chunk_shared_selection(q[::-1], pos, kbar, E, 5, 2) == base
    assert O.chunk_shared_selection(np.concatenate([q, q]), pos, kbar, E, 5, 2) == base


def test_shared_selection_candidates_from_the_first_row():
    kbar, E, q = _shared_case(4, n_query=3)
    gq, ge, S = O.chunk_shared_selection(q, 64 * 5 + 63, kbar, E, 4, 4)
    assert max(S) < 5 and len(S) == 5                  # all 5 candidates, fewer than the budget
    assert O.chunk_shared_selection(q, -1, kbar, E, 4, 4) == ([], [], [])


# --------------------------------------------------------------- selection
def test_selection_fixture():
    for case in _golden("selection_small.json")["cases"]:
        n = len(case["s_q"])
        gq, ge, S = O.select_blocks(case["s_q"], case["E"], n, case["kq"], case["ke"])
        assert gq == case["gamma_q"] and ge == case["gamma_e"] and S == case["S"]


def _brute_topk(scores, k):
    n = len(scores)
    k = min(k, n)
    best = None
    for comb in itertools.combinations(range(n), k):
        tot = sum(scores[j] for j in comb)          # integers: exact sums
        key = (-tot, comb)                           # then lexicographically smallest ids
        if best is None or key < best:
            best = key
    return list(best[1])


@pytest.mark.parametrize("seed", range(40))
def test_top_blocks_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 13))
    scores = [int(v) for v in rng.integers(-3, 4, size=n)]    # many ties
    k = int(rng.integers(0, n + 2))
    assert sorted(O.top_blocks(scores, k)) == _brute_topk(scores, k)


# --------------------------------------------------------------- attention
def _sdpa(q, k, v):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None, :, None, :],
        torch.from_numpy(k.astype(np.float64))[None, None].expand(1, q.shape[0], -1, -1),
        torch.from_numpy(v.astype(np.float64))[None, None].expand(1, q.shape[0], -1, -1))
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("pos", [64 * 5, 64 * 5 + 17, 64 * 9 - 1])
def test_dense_equivalence_when_topk_covers_all_blocks(pos):
    rng = np.random.default_rng(pos)
    T = pos + 1
    D = 32
    K = rng.standard_normal((T, D)).astype(np.float32)
    V = rng.standard_normal((T, D)).astype(np.float32)
    q = rng.standard_normal((3, D)).astype(np.float32)
    c = pos // 64
    lam = rng.standard_normal(T).astype(np.float32)
    kbar = O.subblock_key_means(K, False)
    E = O.block_eviction_scores(O.subblock_logit_means(lam))
    s = O.query_block_scores(q, kbar, c)
    _, _, S = O.select_blocks(s, E, c, kq=c, ke=0)
    assert S == list(range(c))
    got = O.sparse_attention(q, K, V, S, pos)
    np.testing.assert_allclose(got, _sdpa(q, K[:T], V[:T]), rtol=1e-12, atol=1e-12)


def test_window_only_attention():
    rng = np.random.default_rng(7)
    pos = 64 * 6 + 20
    K = rng.standard_normal((pos + 1, 16)).astype(np.float32)
    V = rng.standard_normal((pos + 1, 16)).astype(np.float32)
    q = rng.standard_normal((2, 16)).astype(np.float32)
    got = O.sparse_attention(q, K, V, [], pos)
    np.testing.assert_allclose(got, _sdpa(q, K[64 * 6:], V[64 * 6:]), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_attended_values():
    rng = np.random.default_rng(8)
    pos = 64 * 7 + 3
    K = rng.standard_normal((pos + 1, 8)).astype(np.float32)
    V = rng.standard_normal((pos + 1, 8)).astype(np.float32)
    S = [1, 4]
    got = O.sparse_attention(np.zeros((1, 8), np.float32), K, V, S, pos)
    rows = list(range(64, 128)) + list(range(256, 320)) + list(range(448, pos + 1))
    np.testing.assert_allclose(got[0], V[rows].astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-13)


def test_one_hot_values_give_softmax_weights():
    rng = np.random.default_rng(9)
    pos = 64 * 2 + 5          # attended: block 0 + window of 6 tokens = 70 tokens
    D = 16
    K = rng.standard_normal((pos + 1, D)).astype(np.float32)
    idx = list(range(0, 64)) + list(range(128, pos + 1))
    V = np.zeros((pos + 1, len(idx)), np.float32)
    for j, t in enumerate(idx):
        V[t, j] = 1.0
    q = rng.standard_normal((1, D)).astype(np.float32)
    got = O.sparse_attention(q, K, V, [0], pos)[0]
    logits = torch.from_numpy(K[idx].astype(np.float64)) @ torch.from_numpy(q[0].astype(np.float64)) / math.sqrt(D)
    np.testing.assert_allclose(got, torch.softmax(logits, 0).numpy(), rtol=1e-12, atol=1e-15)


# ----------------------------------------------------- eviction & locality
@pytest.mark.parametrize("kq,ke,L", [(4, 4, 64 * 20 + 13), (2, 6, 64 * 12 + 50), (8, 8, 64 * 30 + 1), (6, 3, 64 * 17)])
def test_eviction_rule_and_locality_bound(kq, ke, L):
    w = NI.scaled(NI.WORKLOADS["tiny"], prompt_len=L, n_steps=320, kq=kq, ke=ke, head_dim=16)
    K, V, lam = NI.unit_kv(w, 0, 0)
    q = NI.queries(w)[:, 0]                        # [n, Hq=G, D]
    tr = O.decode_unit(K, V, lam, q, w.positions(), kq, ke, bf16=False, attend=False)
    k = kq + ke
    dropped = set()
    for t in range(len(tr.sel)):
        ge = set(tr.gamma_e[t])
        assert not (ge & dropped), f"eviction rule broken at step {t}"
        if t > 0:
            dropped |= set(tr.gamma_e[t - 1]) - ge
            c = int(w.positions()[t]) // 64
            if c >= ke:
                assert tr.locality[t] >= ke / k - 1e-12
    # the run must cross several block boundaries
    assert int(w.positions()[-1]) // 64 - int(w.positions()[0]) // 64 >= 4


def test_locality_counts_previous_window_as_held():
    assert O.locality([1, 2, 3], 7, [2, 3, 7, 9]) == 0.75
    assert O.locality([], 0, []) == 1.0


# ---------------------------------------------------------------- the pool
def _pool_sequences():
    g = _golden("pool_lru.json")
    yield "first", g["n_slots"], g["steps"]
    for i, seq in enumerate(g["sequences"]):
        yield f"seq{i}", seq["n_slots"], seq["steps"]


@pytest.mark.parametrize("name,n_slots,steps", list(_pool_sequences()), ids=[s[0] for s in _pool_sequences()])
def test_pool_fixture(name, n_slots, steps):
    pool = O.BlockPool(n_slots)
    for st in steps:
        misses, ins, phys = pool.step(st["t"], st["S"], st["insert"])
        assert [list(m) for m in misses] == st["misses"], st
        assert ins == st["insert_slot"] and phys == st["phys"], st
        # the pool holds every block of S, each in the slot phys names
        assert [pool.slot_of(b) for b in sorted(st["S"])] == st["phys"]
        if ins >= 0:
            assert pool.slot_block[ins] == st["insert"]


def test_pool_fixture_covers_the_insert_cases():
    """The hand-worked sequences include an insert evicted by a miss of the same
    step, an insert of a block already resident and an insert selected in the
    same step."""
    seqs = list(_pool_sequences())
    evicted = resident = selected = False
    for _, n_slots, steps in seqs:
        pool = O.BlockPool(n_slots)
        for st in steps:
            before = pool.resident()
            pool.step(st["t"], st["S"], st["insert"])
            if st["insert"] is None:
                continue
            resident |= st["insert"] in before
            evicted |= st["insert"] not in before and st["insert_slot"] < 0
            selected |= st["insert"] in st["S"] and st["insert_slot"] >= 0
    assert evicted and resident and selected


def test_pool_replay_invariants():
    w = NI.scaled(NI.WORKLOADS["tiny"], prompt_len=64 * 24 + 9, n_steps=400, kq=5, ke=6, head_dim=16)
    K, V, lam = NI.unit_kv(w, 0, 0)
    q = NI.queries(w)[:, 0]
    P = 14
    tr = O.decode_unit(K, V, lam, q, w.positions(), 5, 6, bf16=False, pool_slots=P, attend=False)
    resident = {}
    total_misses = inserts = 0
    for t, S in enumerate(tr.sel):
        before = set(resident)
        c = int(w.positions()[t]) // 64
        completed = t > 0 and c > int(w.positions()[t - 1]) // 64
        if completed and tr.insert_slot[t] >= 0:
            slot = tr.insert_slot[t]
            resident = {b: s for b, s in resident.items() if s != slot}
            resident[c - 1] = slot
            inserts += 1
        misses = tr.misses[t]
        assert [b for b, _ in misses] == sorted(set(S) - set(resident))
        for b, s in misses:
            resident = {bb: ss for bb, ss in resident.items() if ss != s}
            resident[b] = s
        total_misses += len(misses)
        assert all(b in resident for b in S)
        assert [resident[b] for b in S] == tr.phys[t]
        assert len(set(resident.values())) == len(resident) <= P
        if completed:
            # the completed block enters the pool unless it was resident already
            # or a miss of the same step took its slot again (reading U13); the
            # pool is larger than k, so in a decode run that last case cannot
            # happen: the block is always resident after the step
            assert tr.insert_slot[t] >= 0 or (c - 1) in before
            assert resident.get(c - 1, -1) >= 0
            if tr.insert_slot[t] >= 0:
                assert resident[c - 1] == tr.insert_slot[t]
        else:
            assert tr.insert_slot[t] == -1
    assert total_misses > 0 and inserts > 0


def test_pool_restart_mid_run():
    """A restart at step r forgets every resident block: step r misses every
    selected block (ascending, into the lowest slots, after the completed block
    when one is inserted first), the selections and outputs are unchanged, the
    steps before r are unchanged, and from r on the trace equals a pool replay
    that starts empty at r."""
    w = NI.scaled(NI.WORKLOADS["tiny"], prompt_len=64 * 24 + 60, n_steps=40, kq=5, ke=6, head_dim=16)
    K, V, lam = NI.unit_kv(w, 0, 0)
    q = NI.queries(w)[:, 0]
    pos = w.positions()
    P, r = 14, 7                                   # a block completes at step 4
    a = O.decode_unit(K, V, lam, q, pos, 5, 6, bf16=False, pool_slots=P)
    b = O.decode_unit(K, V, lam, q, pos, 5, 6, bf16=False, pool_slots=P, pool_reset_at=r)
    assert a.sel == b.sel and all(np.array_equal(x, y) for x, y in zip(a.out, b.out))
    assert a.misses[:r] == b.misses[:r] and a.phys[:r] == b.phys[:r]
    assert [m for m, _ in b.misses[r]] == b.sel[r] and [s for _, s in b.misses[r]] == list(range(len(b.sel[r])))
    assert sum(map(len, b.misses)) > sum(map(len, a.misses))
    pool = O.BlockPool(P)
    for t in range(r, len(pos)):
        c, c0 = int(pos[t]) // 64, int(pos[t - 1]) // 64
        m, ins, ph = pool.step(t, b.sel[t], c0 if c > c0 else None)
        assert (m, ins, ph) == (b.misses[t], b.insert_slot[t], b.phys[t])
    # a restart on the step a block completes: the inserted block takes slot 0
    c = pos // 64
    r2 = int(np.nonzero(c[1:] > c[:-1])[0][0]) + 1
    d = O.decode_unit(K, V, lam, q, pos, 5, 6, bf16=False, pool_slots=P, attend=False, pool_reset_at=r2)
    assert d.insert_slot[r2] == 0
    assert [s for _, s in d.misses[r2]] == list(range(1, 1 + len(d.misses[r2])))
    assert [m for m, _ in d.misses[r2]] == [j for j in d.sel[r2] if j != c[r2] - 1]


# ---------------------------------------------------------------- eviction head
def test_softplus_closed_forms():
    # log 2 at 0; x + log1p(e^-x) and log1p(e^x) written out with the math module
    assert O.softplus(0.0) == math.log(2.0)
    for x in (-40.0, -3.5, -1e-3, 0.7, 5.0, 35.0, 800.0):
        ref = x + math.log1p(math.exp(-x)) if x > 0 else math.log1p(math.exp(x))
        assert abs(float(O.softplus(x)) - ref) <= 1e-15 * max(1.0, abs(ref))


def test_eviction_head_brute_force():
    """Eq. 4 term by term in plain Python on a tiny head."""
    rng = np.random.default_rng(4)
    T, D, De = 5, 6, 3
    V = rng.standard_normal((T, D))
    W1 = rng.standard_normal((D, De))
    W2 = rng.standard_normal(De)
    got = O.eviction_logits(V, W1, W2)
    for t in range(T):
        s = 0.0
        for j in range(De):
            h = sum(V[t, d] * W1[d, j] for d in range(D))
            s += math.log1p(math.exp(h)) * W2[j] if h < 30 else (h + math.log1p(math.exp(-h))) * W2[j]
        assert abs(got[t] - s) <= 1e-12 * max(1.0, abs(s))


def test_eviction_head_special_weights():
    rng = np.random.default_rng(5)
    V = rng.standard_normal((7, 8))
    W2 = rng.standard_normal(8)
    # W1 = 0: every token scores log(2) * sum(W2)
    assert np.allclose(O.eviction_logits(V, np.zeros((8, 8)), W2), math.log(2.0) * W2.sum(), rtol=0, atol=1e-14)
    # W1 = I, W2 = e_i: the softplus of dimension i
    for i in (0, 5):
        e = np.zeros(8)
        e[i] = 1.0
        assert np.allclose(O.eviction_logits(V, np.eye(8), e), [math.log1p(math.exp(v)) for v in V[:, i]],
                           rtol=1e-15, atol=0)
    # linear in W2
    Wa, Wb = rng.standard_normal(8), rng.standard_normal(8)
    W1 = rng.standard_normal((8, 8))
    assert np.allclose(O.eviction_logits(V, W1, Wa + Wb),
                       O.eviction_logits(V, W1, Wa) + O.eviction_logits(V, W1, Wb), rtol=1e-12, atol=1e-12)


# ---------------------------------------------- alternative readings (U21, U22)
def _rank_order(E, ids):
    """ids ordered by (E desc, id asc), the order of Eq. 7's top-k."""
    return sorted(ids, key=lambda j: (-float(E[j]), j))


def test_fill_remaining_brute_force():
    """U21 on tiny inputs: Gamma_q is the default one, the query-agnostic part
    is the unique subset of the candidates outside Gamma_q that precedes all
    the others in (E desc, id asc) order (found by enumerating every subset),
    and the union holds exactly min(kq + ke, c) blocks."""
    rng = np.random.default_rng(21)
    for trial in range(300):
        c = int(rng.integers(0, 11))
        s_q = rng.integers(-3, 4, size=c).astype(np.float64)       # many ties
        E = rng.integers(-2, 3, size=c).astype(np.float32)
        kq, ke = int(rng.integers(0, 6)), int(rng.integers(0, 6))
        g_q, g_f, S = O.select_blocks_fill(s_q, E, c, kq, ke)
        assert g_q == O.select_blocks(s_q, E, c, kq, ke)[0]
        rest = [j for j in range(c) if j not in set(g_q)]
        n_e = min(ke, len(rest))
        assert len(g_f) == n_e and not set(g_f) & set(g_q)
        assert len(S) == min(kq + ke, c) and S == sorted(set(g_q) | set(g_f))
        pos = {j: i for i, j in enumerate(_rank_order(E, rest))}
        winners = [set(R) for R in itertools.combinations(rest, n_e)
                   if all(pos[a] < pos[b] for a in R for b in rest if b not in R)]
        assert winners == [set(g_f)], (trial, c, kq, ke)


def test_fill_remaining_reduces_to_one_budget():
    rng = np.random.default_rng(22)
    for _ in range(50):
        c = int(rng.integers(1, 40))
        s_q, E = rng.standard_normal(c), rng.standard_normal(c).astype(np.float32)
        k = int(rng.integers(0, 12))
        assert O.select_blocks_fill(s_q, E, c, 0, k)[2] == O.select_blocks(s_q, E, c, 0, k)[2]
        assert O.select_blocks_fill(s_q, E, c, k, 0)[2] == O.select_blocks(s_q, E, c, k, 0)[2]


def test_readmissions_counts_returns_to_the_query_agnostic_part():
    # worked by hand: block 2 leaves at step 1 and returns at step 2; block 5
    # leaves at step 2 and returns at step 4 after one step away, then leaves
    # and returns again at step 6
    seq = [[1, 2, 5], [0, 1, 5], [1, 2], [1, 3], [1, 5], [1, 6], [1, 5]]
    assert O.readmissions(seq) == 3
    assert O.readmissions([[1, 2], [1, 2], [2, 3], [3, 4]]) == 0
    assert O.readmissions([]) == 0


def test_fill_remaining_can_break_the_eviction_rule():
    """Hand-worked: E = [10, 9, 8, 7] over four fixed candidates, kq = 1,
    ke = 2.  The query picks block 0, then block 3, then block 0 again.
    Under U21 the query-agnostic part is {1, 2}, {0, 1}, {1, 2}: block 2 is
    dropped at step 1 and re-admitted at step 2.  Under U1 it is {0, 1}
    every step."""
    E = np.float32([10, 9, 8, 7])
    picks = [0, 3, 0]
    parts_fill, parts_union = [], []
    for p in picks:
        s_q = np.zeros(4)
        s_q[p] = 1.0
        parts_fill.append(O.select_blocks_fill(s_q, E, 4, 1, 2)[1])
        parts_union.append(O.select_blocks(s_q, E, 4, 1, 2)[1])
    assert parts_fill == [[1, 2], [0, 1], [1, 2]]
    assert parts_union == [[0, 1]] * 3
    assert O.readmissions(parts_fill) == 1 and O.readmissions(parts_union) == 0


def test_fill_remaining_readmits_in_decode_runs_and_union_never_does():
    w = NI.scaled(NI.WORKLOADS["tiny"], prompt_len=64 * 20 + 5, n_steps=200, kq=4, ke=4, head_dim=16, rho=0.9)
    K, V, lam = NI.unit_kv(w, 0, 0)
    q = NI.queries(w)[:, 0]
    union = O.decode_unit(K, V, lam, q, w.positions(), 4, 4, bf16=False, attend=False)
    fill = O.decode_unit(K, V, lam, q, w.positions(), 4, 4, bf16=False, attend=False, fill_remaining=True)
    assert O.readmissions(union.gamma_e) == 0
    assert O.readmissions(fill.gamma_e) > 0
    for t, p in enumerate(w.positions()):
        c = int(p) // 64
        assert len(fill.sel[t]) == min(8, c) and len(union.sel[t]) <= min(8, c)


def test_evict_bias_zero_and_constant_change_nothing():
    rng = np.random.default_rng(23)
    T, D, pos = 64 * 5 + 9, 16, 64 * 5 + 8
    K, V = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    q = rng.standard_normal((3, D))
    S = [0, 2, 3]
    ref = O.sparse_attention(q, K, V, S, pos)
    assert np.array_equal(O.sparse_attention(q, K, V, S, pos, np.zeros(T)), ref)
    # softmax is invariant to adding one constant to every logit
    np.testing.assert_allclose(O.sparse_attention(q, K, V, S, pos, np.full(T, -7.25)), ref, rtol=1e-12, atol=1e-13)


def test_evict_bias_brute_force():
    """U22 term by term in plain Python on a tiny case."""
    rng = np.random.default_rng(24)
    T, D, pos = 64 * 2 + 3, 4, 64 * 2 + 2
    K, V = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    lam = rng.standard_normal(T) * 2
    q = rng.standard_normal((2, D))
    S = [1]
    got = O.sparse_attention(q, K, V, S, pos, lam)
    toks = list(range(64, 128)) + list(range(128, pos + 1))
    for g in range(2):
        ls = [sum(q[g, d] * K[i, d] for d in range(D)) / math.sqrt(D) + lam[i] for i in toks]
        m = max(ls)
        ws = [math.exp(l - m) for l in ls]
        z = sum(ws)
        for d in range(D):
            ref = sum(w * V[i, d] for w, i in zip(ws, toks)) / z
            assert abs(got[g, d] - ref) <= 1e-12


def test_evict_bias_can_pick_one_token():
    rng = np.random.default_rng(25)
    T, D, pos = 64 * 3 + 1, 8, 64 * 3
    K, V = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    q = rng.standard_normal((1, D))
    lam = np.full(T, -1e4)
    lam[70] = 0.0
    np.testing.assert_allclose(O.sparse_attention(q, K, V, [1], pos, lam)[0], V[70], rtol=0, atol=1e-12)
