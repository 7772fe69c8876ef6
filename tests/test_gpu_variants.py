"""Parity of the two variant calls with the oracle's alternative readings:
nosa_select_blocks_fill (reading U21 of Eq. 7) and nosa_sparse_decode_attn_bias
(reading U22 of ED-DMA).  Same bars as the main path: sets exact up to
accepted score ties, outputs within 2e-2 (bf16) or 1e-4 (fp32)."""
import itertools

import numpy as np
import pytest
import torch

import nosa_inputs as NI
from kv_cache_offload_amd import binding as nb
from kv_cache_offload_amd import runner as R
from oracle import nosa_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nb.load()
    yield
    torch.cuda.synchronize()


def _banner(msg):
    print(f"\n[case] {msg}", flush=True)


def fill_ok(S_gpu, s_q, E, c, kq, ke, rel=H.REL_TIE) -> bool:
    """S_gpu is Gamma_q' U F(Gamma_q') for some top-kq set Gamma_q' of s_q once
    scores within `rel` of the kq-th best count as equal, with F the top-ke
    of E over the candidates outside Gamma_q' (E is bit-exact: no allowance)."""
    S = sorted(int(x) for x in S_gpu)
    kk = min(kq, c)
    if kk == 0:
        return S == O.select_blocks_fill(s_q, E, c, kq, ke)[2]
    order = O.top_blocks(list(s_q[:c]), c)
    thr = float(s_q[order[kk - 1]])
    tie = [j for j in range(c) if abs(float(s_q[j]) - thr) <= rel * max(abs(float(s_q[j])), abs(thr))]
    must = [j for j in range(c) if float(s_q[j]) > thr and j not in tie]
    for extra in itertools.combinations(tie, kk - len(must)):
        g_q = set(must) | set(extra)
        rest = [j for j in range(c) if j not in g_q]
        g_f = [rest[i] for i in O.top_blocks([E[j] for j in rest], ke)]
        if sorted(g_q | set(g_f)) == S:
            return True
    return False


SEL_CASES = [
    ("boundaries", dict(batch=3, prompt_len=64 * 40 + 50, n_steps=90), 1),
    ("short-context", dict(batch=2, prompt_len=64 * 30 + 3, n_steps=12, kq=16, ke=48), 1),
    ("kq-only", dict(batch=2, prompt_len=64 * 90 + 9, n_steps=6, kq=7, ke=0), 1),
    ("ke-only", dict(batch=2, prompt_len=64 * 90 + 9, n_steps=6, kq=0, ke=9), 1),
    ("layer32k-heads", dict(batch=2, prompt_len=64 * 512 + 5, n_steps=4), 1),
    ("many-rows", dict(batch=2, prompt_len=64 * 300 + 40, n_steps=8), 8),
]


@pytest.mark.parametrize("name,over,n_query", SEL_CASES, ids=[c[0] for c in SEL_CASES])
def test_select_fill_matches_oracle(name, over, n_query):
    _banner(f"select fill {name}")
    w = NI.scaled(NI.WORKLOADS["layer32k"], **over)
    K, V, lam, q = NI.layer_inputs(w)
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    positions = w.positions()
    L.pool_blocks(kv, logits, 0, int(positions[-1]) // 64)
    G, k = w.group, w.kq + w.ke
    E = {(b, h): O.block_eviction_scores(O.subblock_logit_means(lam[b, h]))
         for b in range(w.batch) for h in range(w.n_kv_heads)}
    kbar = {(b, h): O.subblock_key_means(K[b, h], True) for b in range(w.batch) for h in range(w.n_kv_heads)}
    steps = range(0, w.n_steps, n_query)
    for t0 in steps:
        rows = list(range(t0, min(w.n_steps, t0 + n_query)))
        nq = len(rows)
        qr = qd[rows].permute(1, 0, 2, 3).contiguous()               # [B, n_query, Hq, D]
        pr = pos[rows].t().contiguous()                              # [B, n_query]
        sel = torch.full((w.batch, nq, w.n_kv_heads, max(k, 1)), -1, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros((w.batch, nq, w.n_kv_heads), dtype=torch.int32, device="cuda")
        ws = torch.zeros(nb.workspace_size(L.dims, nb.OP_SELECT, nq, w.kq, w.ke), dtype=torch.uint8, device="cuda")
        nb.select_blocks_fill(L.dims, qr, nq, pr, L.k_comp, L.e_blk, w.kq, w.ke, sel, n_sel, ws)
        torch.cuda.synchronize()
        S_all, N_all = sel.cpu().numpy(), n_sel.cpu().numpy()
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                for r, t in enumerate(rows):
                    c = int(positions[t]) // 64
                    S = list(S_all[b, r, h, : N_all[b, r, h]])
                    assert S == sorted(S) and all(x == -1 for x in S_all[b, r, h, N_all[b, r, h]:])
                    assert len(S) == min(k, c)
                    s_q = O.query_block_scores(q[t, b, h * G:(h + 1) * G], kbar[b, h], c)
                    ok = S == O.select_blocks_fill(s_q, E[b, h], c, w.kq, w.ke)[2] or \
                        fill_ok(S, s_q, E[b, h], c, w.kq, w.ke)
                    assert ok, (name, b, h, t)


def test_select_fill_exact_ties():
    """Keys and eviction logits repeating three block patterns: every budget
    is filled from groups of equal scores, broken by block id on both sides
    with no allowance."""
    _banner("select fill, exact ties")
    w = NI.scaled(NI.WORKLOADS["layer32k"], batch=2, prompt_len=64 * 60 + 40, n_steps=6)
    K, V, lam, q = NI.layer_inputs(w)
    rng = np.random.default_rng(7)
    pat = torch.from_numpy(rng.standard_normal((3, w.head_dim)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    blk = np.arange(K.shape[2]) // 64
    K[:] = pat[blk % 3][None, None]
    lam[:] = np.float32([0.5, -1.0, 2.0])[(blk * 7 // 3) % 3][None, None]
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    L.pool_blocks(kv, logits, 0, int(w.positions()[0]) // 64)
    G = w.group
    for t in range(w.n_steps):
        L.select(qd[t], pos[t], fill=True)
        torch.cuda.synchronize()
        S_all, N_all = L.sel.cpu().numpy(), L.n_sel.cpu().numpy()
        c = int(w.positions()[t]) // 64
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                kbar = O.subblock_key_means(K[b, h], True)
                E = O.block_eviction_scores(O.subblock_logit_means(lam[b, h]))
                s_q = O.query_block_scores(q[t, b, h * G:(h + 1) * G], kbar, c)
                assert list(S_all[b, h, : N_all[b, h]]) == O.select_blocks_fill(s_q, E, c, w.kq, w.ke)[2]


BIAS_CASES = [
    ("bf16-D128", dict(batch=2, prompt_len=64 * 70 + 33, n_steps=40)),           # crosses a block end
    ("bf16-D64-G4", dict(batch=2, prompt_len=64 * 50 + 5, n_steps=6, head_dim=64, n_q_heads=8)),
    ("fp32-tiny", None),
]


@pytest.mark.parametrize("name,over", BIAS_CASES, ids=[c[0] for c in BIAS_CASES])
def test_attention_bias_matches_oracle(name, over):
    """The biased attention over the oracle's own selections (injected), every
    unit and step, against the oracle's softmax(q K^T / sqrt(D) + lambda)."""
    _banner(f"attention bias {name}")
    w = NI.WORKLOADS["tiny"] if over is None else NI.scaled(NI.WORKLOADS["layer32k"], **over)
    K, V, lam, q = NI.layer_inputs(w)
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    G, k, bf16 = w.group, w.kq + w.ke, w.dtype == "bf16"
    trs = {(b, h): O.decode_unit(K[b, h], V[b, h], lam[b, h], q[:, b, h * G:(h + 1) * G], w.positions(), w.kq, w.ke,
                                 bf16=bf16, evict_bias=True)
           for b in range(w.batch) for h in range(w.n_kv_heads)}
    err = 0.0
    for t in range(w.n_steps):
        sel = np.full((w.batch, w.n_kv_heads, max(k, 1)), -1, np.int32)
        n_sel = np.zeros((w.batch, w.n_kv_heads), np.int32)
        for (b, h), tr in trs.items():
            sel[b, h, : len(tr.sel[t])] = tr.sel[t]
            n_sel[b, h] = len(tr.sel[t])
        L.sel.copy_(torch.from_numpy(sel))
        L.n_sel.copy_(torch.from_numpy(n_sel))
        L.attend_resident_bias(qd[t], kv, pos[t], logits)
        torch.cuda.synchronize()
        out = L.out.float().cpu().numpy()
        for (b, h), tr in trs.items():
            e = float(np.max(np.abs(out[b, h * G:(h + 1) * G] - tr.out[t])))
            err = max(err, e)
            assert e <= H.ATOL[w.dtype], (name, b, h, t, e)
    print(f"max |err| {err:.3g}", flush=True)


def test_attention_bias_of_zero_is_the_plain_attention():
    _banner("attention bias of zero")
    w = NI.scaled(NI.WORKLOADS["layer32k"], batch=2, prompt_len=64 * 40 + 17, n_steps=3)
    K, V, lam, q = NI.layer_inputs(w)
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    L.pool_blocks(kv, logits, 0, int(w.positions()[0]) // 64)
    zero = torch.zeros_like(logits)
    for t in range(w.n_steps):
        L.select(qd[t], pos[t])
        L.attend_resident(qd[t], kv, pos[t])
        torch.cuda.synchronize()
        ref = L.out.clone()
        L.attend_resident_bias(qd[t], kv, pos[t], zero)
        torch.cuda.synchronize()
        assert float((L.out.float() - ref.float()).abs().max()) <= 1e-3
