"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: pooled keys and eviction scores bit-exact; selected block sets equal
to the oracle's except where two scores at the kq-th place lie within 1e-5
relative (then the GPU's choice must be a valid top-kq, and the oracle
continues with it); pool tables, miss lists and slots exact; attention
outputs within 2e-2 absolute (bf16) or 1e-4 (fp32).
"""
import math
import os

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


def _w(base, **kw):
    return NI.scaled(NI.WORKLOADS[base], **kw)


# ------------------------------------------------------------- pool keys
@pytest.mark.parametrize("dtype,D,G", [("f32", 64, 2), ("bf16", 128, 8), ("bf16", 64, 4), ("f32", 128, 16)])
def test_pool_keys_bit_exact(dtype, D, G):
    _banner(f"pool_keys {dtype} D={D} G={G}")
    w = _w("layer32k", batch=2, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, prompt_len=64 * 37 + 5,
           n_steps=1, dtype=dtype)
    K, V, lam, q = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, q)
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, D, w.n_blocks, dtype, 4, 4)
    layer.k_comp.fill_(float("nan"))
    layer.e_sub.fill_(float("nan"))
    layer.e_blk.fill_(float("nan"))
    layer.pool_blocks(kv, logits, 0, 20)
    layer.pool_blocks(kv, logits, 20, 37)
    kc = layer.k_comp.float().cpu().numpy()
    es = layer.e_sub.cpu().numpy()
    eb = layer.e_blk.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            kbar = O.subblock_key_means(K[b, h], bf16=(dtype == "bf16"))[: 37 * 4]
            esub = O.subblock_logit_means(lam[b, h])[: 37 * 4]
            E = O.block_eviction_scores(esub)
            np.testing.assert_array_equal(kc[b, h, : 37 * 4].view(np.uint32), kbar.view(np.uint32))
            np.testing.assert_array_equal(es[b, h, : 37 * 4].view(np.uint32), esub.view(np.uint32))
            np.testing.assert_array_equal(eb[b, h, :37].view(np.uint32), E.view(np.uint32))
            assert np.all(np.isnan(kc[b, h, 37 * 4:])) and np.all(np.isnan(eb[b, h, 37:]))


def test_pool_keys_from_window_buffer():
    _banner("pool_keys from a one-block window buffer")
    w = _w("layer32k", batch=2, prompt_len=64 * 9, n_steps=1)
    K, V, lam, q = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, q)
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, 4, 4)
    ref = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, 4, 4)
    ref.pool_blocks(kv, logits, 6, 7)
    window = kv[:, :, 6].clone()
    layer.pool_window(window, logits, 6)
    assert torch.equal(layer.k_comp.view(torch.int16), ref.k_comp.view(torch.int16))
    assert torch.equal(layer.e_blk, ref.e_blk)


# --------------------------------------------------------------- selection
SELECT_CASES = [
    # name, workload overrides, kq, ke, positions
    ("f32 D64 G2", dict(dtype="f32", head_dim=64, n_q_heads=2, n_kv_heads=1), 4, 4,
     [5, 64 * 3 + 1, 64 * 37 + 17, 64 * 80 - 1]),
    ("bf16 D128 G8", dict(), 16, 48, [0, 64 * 10 + 3, 64 * 70, 64 * 200 + 63]),
    ("bf16 D64 G4 kq only", dict(head_dim=64, n_q_heads=8), 12, 0, [64 * 50 + 9, 64 * 129]),
    ("bf16 D128 G16 ke only", dict(n_q_heads=32), 0, 20, [64 * 33 + 40]),
    ("bf16 D128 wide k", dict(), 100, 150, [64 * 300 + 2]),
    ("bf16 D128 split scan", dict(), 16, 48, [64 * 1100 + 5, 64 * 700 + 1]),
    ("f32 D128 split scan", dict(dtype="f32", n_q_heads=4), 5, 7, [64 * 1030 + 63]),
]


@pytest.mark.parametrize("name,over,kq,ke,positions", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_matches_oracle(name, over, kq, ke, positions):
    _banner(f"select {name}")
    T = max(positions) + 1
    w = _w("layer32k", batch=3, prompt_len=T, n_steps=1, kq=kq, ke=ke, prefill=True, **over)
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, kq, ke)
    layer.pool_blocks(kv, logits, 0, T // 64)
    rng = np.random.default_rng(11)
    ties = 0
    for p in positions:
        qn = rng.standard_normal((w.batch, w.n_q_heads, w.head_dim)).astype(np.float32)
        if w.dtype == "bf16":
            qn = NI.round_to_bf16(qn)
        qd = torch.from_numpy(qn).cuda().to(R.torch_dtype(w.dtype))
        pos = torch.full((w.batch,), p, dtype=torch.int32, device="cuda")
        layer.select(qd, pos)
        sel = layer.sel.cpu().numpy()
        n = layer.n_sel.cpu().numpy()
        c = p // 64
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                kbar = O.subblock_key_means(K[b, h], bf16=(w.dtype == "bf16"))
                E = O.block_eviction_scores(O.subblock_logit_means(lam[b, h]))
                s_q = O.query_block_scores(qn[b, h * w.group:(h + 1) * w.group], kbar, c)
                _, _, S = O.select_blocks(s_q, E, c, kq, ke)
                got = list(sel[b, h, : n[b, h]])
                assert np.all(sel[b, h, n[b, h]:] == -1)
                if got != S:
                    assert H.selection_ok(got, s_q, E, c, kq, ke), (p, b, h, got, S)
                    ties += 1
    assert ties <= 2


def test_select_invalid_positions_give_empty_sets():
    _banner("select with out-of-range positions")
    w = _w("layer32k", batch=2, prompt_len=64 * 8, n_steps=1, prefill=True)
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, 2, 2)
    layer.pool_blocks(kv, logits, 0, 8)
    q = torch.randn(w.batch, w.n_q_heads, w.head_dim, device="cuda").to(torch.bfloat16)
    pos = torch.tensor([-5, 64 * 8 + 10], dtype=torch.int32, device="cuda")
    layer.select(q, pos)
    assert torch.all(layer.n_sel == 0) and torch.all(layer.sel == -1)
    # the workspace is left ready: a valid call right after works
    pos = torch.tensor([64 * 7 + 3, 64 * 7 + 3], dtype=torch.int32, device="cuda")
    layer.select(q, pos)
    assert torch.all((layer.n_sel >= 2) & (layer.n_sel <= 4))   # union of two 2-sets


# --------------------------------------------------------------- attention
ATTN_CASES = [
    ("f32 D64 G2", dict(dtype="f32", head_dim=64, n_q_heads=2, n_kv_heads=1), 8),
    ("bf16 D128 G8", dict(), 64),
    ("bf16 D64 G4", dict(head_dim=64, n_q_heads=8), 12),
    ("bf16 D128 G16", dict(n_q_heads=32), 20),
    ("f32 D128 G1", dict(dtype="f32", n_q_heads=2), 9),
]


@pytest.mark.parametrize("name,over,k", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_with_oracle_selection(name, over, k):
    _banner(f"attention {name}")
    T = 64 * 90 + 1
    w = _w("layer32k", batch=2, prompt_len=T, n_steps=1, prefill=True, **over)
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, k, 0)
    rng = np.random.default_rng(5)
    G = w.group
    for p in (64 * 89 + 0, 64 * 89 + 33, 64 * 90, 64 * 88 + 63, 40):
        c = p // 64
        qn = rng.standard_normal((w.batch, w.n_q_heads, w.head_dim)).astype(np.float32)
        if w.dtype == "bf16":
            qn = NI.round_to_bf16(qn)
        sel = np.full((w.batch, w.n_kv_heads, k), -1, np.int32)
        nsel = np.zeros((w.batch, w.n_kv_heads), np.int32)
        chosen = {}
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                m = int(rng.integers(0, min(k, c) + 1)) if (b + h) % 3 else min(k, c)
                S = sorted(rng.choice(c, size=m, replace=False).tolist()) if m else []
                sel[b, h, :m] = S
                nsel[b, h] = m
                chosen[b, h] = S
        layer.sel.copy_(torch.from_numpy(sel))
        layer.n_sel.copy_(torch.from_numpy(nsel))
        qd = torch.from_numpy(qn).cuda().to(R.torch_dtype(w.dtype))
        pos = torch.full((w.batch,), p, dtype=torch.int32, device="cuda")
        layer.attend_resident(qd, kv, pos)
        out = layer.out.float().cpu().numpy()
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                ref = O.round_output(O.sparse_attention(qn[b, h * G:(h + 1) * G], K[b, h], V[b, h],
                                                        chosen[b, h], p), w.dtype == "bf16")
                err = np.max(np.abs(out[b, h * G:(h + 1) * G] - ref))
                assert err <= H.ATOL[w.dtype], (name, p, b, h, err)


def test_attention_dense_equivalence():
    _banner("attention: all blocks selected equals dense causal attention")
    w = _w("layer32k", batch=1, n_q_heads=8, n_kv_heads=1, prompt_len=64 * 20 + 7, n_steps=1, prefill=True)
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    p = 64 * 20 + 6
    layer = R.DecodeLayer(1, 8, 1, 128, w.n_blocks, "bf16", 20, 0)
    layer.pool_blocks(kv, logits, 0, 20)
    qn = NI.round_to_bf16(np.random.default_rng(2).standard_normal((1, 8, 128)).astype(np.float32))
    qd = torch.from_numpy(qn).cuda().to(torch.bfloat16)
    pos = torch.tensor([p], dtype=torch.int32, device="cuda")
    layer.step_resident(qd, kv, pos)
    assert layer.n_sel.item() == 20
    out = layer.out.float().cpu()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qn[0]).double()[:, None, :],
        torch.from_numpy(K[0, 0, : p + 1]).double()[None].expand(8, -1, -1),
        torch.from_numpy(V[0, 0, : p + 1]).double()[None].expand(8, -1, -1))[:, 0, :]
    assert float((out[0] - ref.float()).abs().max()) <= 2e-2


@pytest.mark.parametrize("fused", [False, True], ids=["separate-calls", "one-launch"])
def test_attention_repeats_are_bit_identical(fused):
    """The same steps run twice give bit-identical sets and outputs; for the
    one-launch step also the same step launched again and again on one
    workspace (each launch with its own flag, the Gamma_e cache reused): the
    final merge combines the partial records in a fixed order whatever order
    the workgroups finish in."""
    _banner(f"determinism across repeats, fused={fused}")
    w = _w("layer32k", batch=4, prompt_len=64 * 100 + 20, n_steps=3)
    K, V, lam, q = NI.layer_inputs(w)
    s1, n1, o1, _ = H.run_resident(w, K, V, lam, q, fused=fused)
    s2, n2, o2, layer = H.run_resident(w, K, V, lam, q, fused=fused)
    for a, b in zip(s1, s2):
        assert np.array_equal(a, b)
    for a, b in zip(o1, o2):
        assert np.array_equal(a, b)
    if fused:
        kv, _, qd, pos = H.device_inputs(w, K, V, lam, q)
        for _ in range(8):
            layer.step_fused(qd[1], kv, pos[1])
            torch.cuda.synchronize()
            assert np.array_equal(layer.sel.cpu().numpy(), s1[1])
            assert np.array_equal(layer.out.float().cpu().numpy(), o1[1])
        assert layer.step_timeouts() == 0


def test_fused_step_under_concurrent_load():
    """The one-launch step while another stream keeps the device busy with
    large products: the step's workgroups then start as the other kernels'
    workgroups leave, not all at once.  Producers never wait, and every
    waiter waits on workgroups of its launch that have started before it or
    are running beside it, so the steps must give the results of an idle
    device bit for bit, with no wait expired."""
    _banner("one-launch step under concurrent load")
    w = _w("layer32k", batch=4, prompt_len=64 * 100 + 20, n_steps=3)
    K, V, lam, q = NI.layer_inputs(w)
    s_ref, _, o_ref, layer = H.run_resident(w, K, V, lam, q, fused=True)
    kv, _, qd, pos = H.device_inputs(w, K, V, lam, q)
    gen = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn(4096, 4096, device="cuda", generator=gen)
    b = torch.randn(4096, 4096, device="cuda", generator=gen)
    side, main = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    sels, outs = [], []
    overlapped = 0
    for _ in range(4):
        side_done = torch.cuda.Event()
        with torch.cuda.stream(side):
            for _ in range(6):
                a = (a @ b) * (1.0 / 64.0)
            side_done.record(side)
        with torch.cuda.stream(main):
            for t in range(w.n_steps):
                layer.step_fused(qd[t], kv, pos[t], main)
                sels.append(layer.sel.clone())
                outs.append(layer.out.clone())
        main.synchronize()
        overlapped += not side_done.query()   # the steps ended while the products still ran
    torch.cuda.synchronize()
    assert overlapped > 0, "the steps never ran beside the products"
    assert torch.isfinite(a).all()
    for i, (s, o) in enumerate(zip(sels, outs)):
        t = i % w.n_steps
        assert np.array_equal(s.cpu().numpy(), s_ref[t]), f"selection differs under load, step {t}"
        assert np.array_equal(o.float().cpu().numpy(), o_ref[t]), f"output differs under load, step {t}"
    assert layer.step_timeouts() == 0


def test_determinism_across_split_counts_and_launch_orders():
    """The same step computed with other work decompositions and launch
    orders: the selected sets must be identical and the outputs agree within
    the output tolerance (bit for bit where the decomposition is the same).

      * attention split count: the same sets in rows of 64, 96 and 200
        entries (9, 13 and 26 splits of 8 blocks per unit);
      * one-launch step worker count: batch 16 (32 units, 8 workers per unit)
        against each entry run alone (2 units, 16 workers per unit); the
        separate calls keep their decomposition per unit, so there the outputs
        are bit-identical;
      * launch order: two layers' steps interleaved on two streams against
        the same steps run one layer after the other;
      * the offload step with the gather on a side stream, on the compute
        stream, and folded into the attention: identical pool tables, miss
        lists and slots."""
    _banner("determinism: split counts, worker counts, launch orders")
    w = _w("layer32k", batch=16, prompt_len=64 * 100 + 20, n_steps=3)
    K, V, lam, q = NI.layer_inputs(w)
    atol = H.ATOL[w.dtype]
    s_ref, n_ref, o_ref, L = H.run_resident(w, K, V, lam, q)
    s_f, n_f, o_f, _ = H.run_resident(w, K, V, lam, q, fused=True)
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    k = w.kq + w.ke
    for t in range(w.n_steps):
        assert np.array_equal(s_f[t], s_ref[t]) and np.array_equal(n_f[t], n_ref[t])
        assert float(np.abs(o_f[t] - o_ref[t]).max()) <= atol
    # attention split counts
    for k_cap in (96, 200):
        ws = torch.zeros(nb.workspace_size(L.dims, nb.OP_ATTN, 1, k_cap, 0), dtype=torch.uint8, device="cuda")
        out = torch.zeros_like(L.out)
        for t in range(w.n_steps):
            sel = torch.full((w.batch, w.n_kv_heads, k_cap), -1, dtype=torch.int32, device="cuda")
            sel[..., :k] = torch.from_numpy(s_ref[t]).cuda()
            n_sel = torch.from_numpy(n_ref[t]).cuda()
            nb.sparse_decode_attn(L.dims, qd[t], kv, L.NB, sel, n_sel, k_cap, kv, L.NB * L.blk_elems, L.blk_elems,
                                  pos[t], None, out, ws)
            torch.cuda.synchronize()
            e = float(np.abs(out.float().cpu().numpy() - o_ref[t]).max())
            assert e <= atol, (k_cap, t, e)
    # worker counts (one-launch step) and grid size (separate calls)
    w1 = NI.scaled(w, batch=1)
    for b in (0, 5, 15):
        sl = slice(b, b + 1)
        s1, n1, o1, _ = H.run_resident(w1, K[sl], V[sl], lam[sl], q[:, sl])
        s1f, n1f, o1f, _ = H.run_resident(w1, K[sl], V[sl], lam[sl], q[:, sl], fused=True)
        for t in range(w.n_steps):
            assert np.array_equal(s1[t][0], s_ref[t][b]) and np.array_equal(s1f[t][0], s_ref[t][b])
            assert np.array_equal(o1[t][0], o_ref[t][b])
            assert float(np.abs(o1f[t][0] - o_ref[t][b]).max()) <= atol
    # launch order: two layers on two streams, steps interleaved
    layers = [R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
              for _ in range(2)]
    c0 = int(w.positions()[0]) // 64
    for Lx in layers:
        Lx.pool_blocks(kv, logits, 0, c0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [[], []]
    for t in range(w.n_steps):
        for i in (1, 0):
            with torch.cuda.stream(streams[i]):
                (layers[i].step_fused if i else layers[i].step_resident)(qd[t], kv, pos[t], streams[i])
                got[i].append((layers[i].sel.clone(), layers[i].out.float().clone()))
    torch.cuda.synchronize()
    for t in range(w.n_steps):
        assert np.array_equal(got[0][t][0].cpu().numpy(), s_ref[t])
        assert np.array_equal(got[1][t][0].cpu().numpy(), s_ref[t])
        assert np.array_equal(got[0][t][1].cpu().numpy(), o_ref[t])
        assert np.array_equal(got[1][t][1].cpu().numpy(), o_f[t])
    # offload with and without the side stream
    wo = _w("offload", batch=3, prompt_len=64 * 40 + 30, n_steps=60, kq=4, ke=6, pool_slots=14)
    Ko, Vo, lamo, qo = NI.layer_inputs(wo)
    ra, _, _ = H.run_offload(wo, Ko, Vo, lamo, qo, side_stream=True)
    for other in (dict(side_stream=False), dict(fused_fetch=True)):
        rb, _, _ = H.run_offload(wo, Ko, Vo, lamo, qo, **other)
        for key in ("sel", "n_sel", "phys", "miss_list", "n_miss", "block_table", "slot_block"):
            for t in range(wo.n_steps):
                assert np.array_equal(ra[key][t], rb[key][t]), (other, key, t)
        for t in range(wo.n_steps):
            assert float(np.abs(ra["out"][t] - rb["out"][t]).max()) <= atol


# ------------------------------------------------------- end-to-end decode
def test_tiny_fp32_decode_matches_oracle():
    _banner("tiny fp32 workload: 16 decode steps")
    w = NI.WORKLOADS["tiny"]
    K, V, lam, q = NI.layer_inputs(w)
    sels, nsels, outs, _ = H.run_resident(w, K, V, lam, q)
    st = H.compare_unit(w, K, V, lam, q, 0, 0, H.unit_selections(sels, nsels, 0, 0), gpu_out=outs)
    assert st["max_err"] <= 1e-4


def test_layer32k_decode_matches_oracle():
    _banner("layer32k workload: B=8, 16/2 heads, D=128, 32K context, 64 steps")
    w = NI.WORKLOADS["layer32k"]
    K, V, lam, q = NI.layer_inputs(w)
    sels, nsels, outs, _ = H.run_resident(w, K, V, lam, q)
    ties = 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            st = H.compare_unit(w, K, V, lam, q, b, h, H.unit_selections(sels, nsels, b, h), gpu_out=outs)
            ties += st["ties"]
    print(f"[layer32k] accepted ties: {ties}", flush=True)


# ------------------------------------------------------------ offload path
def _pool_consistent(layer, host, b, h):
    bt = layer.block_table[b, h].cpu().numpy()
    sb = layer.slot_block[b, h].cpu().numpy()
    for s, blk in enumerate(sb):
        if blk >= 0:
            assert bt[blk] == s
            assert torch.equal(layer.pool[b, h, s].cpu().view(torch.int16), host[b, h, blk].view(torch.int16)), (b, h, s, blk)
    for blk, s in enumerate(bt):
        if s >= 0:
            assert sb[s] == blk


OFFLOAD_MODES = {"side-stream": dict(side_stream=True, fused_fetch=False),
                 "one-stream": dict(side_stream=False, fused_fetch=False), "fused-fetch": dict(fused_fetch=True)}


@pytest.mark.parametrize("mode", list(OFFLOAD_MODES))
def test_offload_small_pool_matches_oracle(mode):
    _banner(f"offload: B=3, L ragged, 100 steps, pool 14 slots, {mode}")
    w = _w("offload", batch=3, prompt_len=64 * 40 + 30, n_steps=100, kq=4, ke=6, pool_slots=14)
    K, V, lam, q = NI.layer_inputs(w)
    rec, layer, host = H.run_offload(w, K, V, lam, q, **OFFLOAD_MODES[mode])
    total = 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            st = H.check_offload_unit(w, K, V, lam, q, rec, b, h)
            total += st["misses"]
            _pool_consistent(layer, host, b, h)
    assert total > w.batch * w.n_kv_heads * 10


@pytest.mark.parametrize("mode", list(OFFLOAD_MODES))
def test_offload_ragged_positions(mode):
    """Batch entries at their own positions (lagging the first by 0, 17, 40
    and 63 tokens), so their windows complete blocks on different steps: each
    completed block is pooled for its entry alone (nosa_pool_keys_entries)
    and inserted for that entry alone (a per-entry insert_block).  Every unit
    against the oracle at its own positions; the compressed keys and eviction
    scores of each entry's complete blocks bit-exact, and nothing written for
    blocks an entry has not completed."""
    _banner(f"offload ragged positions: B=4, lags 0/17/40/63, 100 steps, pool 14, {mode}")
    w = _w("offload", batch=4, prompt_len=64 * 40 + 30, n_steps=100, kq=4, ke=6, pool_slots=14)
    K, V, lam, q = NI.layer_inputs(w)
    offs = [0, 17, 40, 63]
    rec, layer, host = H.run_offload(w, K, V, lam, q, offsets=offs, **OFFLOAD_MODES[mode])
    P = rec["positions"]
    done_steps = [set(np.nonzero(P[1:, b] // 64 > P[:-1, b] // 64)[0] + 1) for b in range(w.batch)]
    assert all(done_steps) and len(set().union(*done_steps)) == sum(map(len, done_steps))   # no two together
    bf16 = w.dtype == "bf16"
    kc = layer.k_comp.float().cpu().numpy()
    es, eb = layer.e_sub.cpu().numpy(), layer.e_blk.cpu().numpy()
    for b in range(w.batch):
        c_end = int(P[-1, b]) // 64
        for h in range(w.n_kv_heads):
            st = H.check_offload_unit(w, K, V, lam, q, rec, b, h)
            assert st["misses"] > 0
            _pool_consistent(layer, host, b, h)
            kbar = O.subblock_key_means(K[b, h], bf16)
            e_sub = O.subblock_logit_means(lam[b, h])
            assert np.array_equal(kc[b, h, : 4 * c_end], kbar[: 4 * c_end])
            assert np.array_equal(es[b, h, : 4 * c_end], e_sub[: 4 * c_end])
            assert np.array_equal(eb[b, h, :c_end], O.block_eviction_scores(e_sub)[:c_end])
            assert not kc[b, h, 4 * c_end:].any() and not eb[b, h, c_end:].any()


def _random_offload_config(seed):
    """A small seeded offload configuration: heads, dtype, budgets, a pool a
    little larger than the selection, ragged per-entry lags, a step form and
    sometimes a cold restart."""
    rng = np.random.default_rng(2000 + seed)
    kq, ke = int(rng.integers(0, 13)), int(rng.integers(0, 13))
    if kq + ke == 0:
        ke = 1
    G, hkv, B = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2])), int(rng.integers(1, 5))
    n_steps = int(rng.integers(20, 121))
    L = int(rng.integers(65 + 64, 4000))
    L += 1 if L % 64 == 0 else 0
    over = dict(batch=B, n_q_heads=G * hkv, n_kv_heads=hkv, head_dim=int(rng.choice([64, 128])),
                dtype=str(rng.choice(["bf16", "f32"])), prompt_len=L, n_steps=n_steps, kq=kq, ke=ke,
                pool_slots=kq + ke + int(rng.integers(1, 21)))
    offsets = [int(x) for x in rng.integers(0, 64, B)]
    mode = str(rng.choice(list(OFFLOAD_MODES)))
    reset_at = int(rng.integers(1, n_steps)) if rng.random() < 0.3 else None
    return over, offsets, mode, reset_at


@pytest.mark.parametrize("seed", range(16))
def test_random_offload_configs_match_oracle(seed):
    """Seeded random offload runs (every step form, ragged lags, pools from
    one to twenty blocks above the selection, both dtypes, head groupings
    1-8, sometimes a cold restart): every unit's sets, misses, slots, tables
    and outputs against the oracle's block pool, and every resident pool
    block byte-identical to its host block."""
    over, offsets, mode, reset_at = _random_offload_config(seed)
    _banner(f"random offload {seed}: {over} lags {offsets} {mode} reset {reset_at}")
    w = _w("offload", **over)
    K, V, lam, q = NI.layer_inputs(w)
    rec, layer, host = H.run_offload(w, K, V, lam, q, offsets=offsets, reset_at=reset_at, **OFFLOAD_MODES[mode])
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            H.check_offload_unit(w, K, V, lam, q, rec, b, h, pool_reset_at=reset_at)
            _pool_consistent(layer, host, b, h)


@pytest.mark.parametrize("reset_at", [30, 34], ids=["mid-block", "on-a-completion"])
def test_offload_cold_restart_mid_run(reset_at):
    """The pool tables cleared before step `reset_at` (every resident block
    forgotten): the same sets, the same outputs within tolerance, more
    misses, and from the restart on the misses, slots and insertions of a
    pool that starts empty there (the oracle's)."""
    _banner(f"offload cold restart at step {reset_at}")
    w = _w("offload", batch=3, prompt_len=64 * 40 + 30, n_steps=60, kq=4, ke=6, pool_slots=14)
    K, V, lam, q = NI.layer_inputs(w)
    base, _, _ = H.run_offload(w, K, V, lam, q)
    rec, layer, host = H.run_offload(w, K, V, lam, q, reset_at=reset_at)
    assert (int(w.positions()[reset_at]) // 64 > int(w.positions()[reset_at - 1]) // 64) == (reset_at == 34)
    for t in range(w.n_steps):
        assert np.array_equal(rec["sel"][t], base["sel"][t]) and np.array_equal(rec["n_sel"][t], base["n_sel"][t])
        assert float(np.abs(rec["out"][t] - base["out"][t]).max()) <= H.ATOL[w.dtype]
    # every selected block misses at the restart, except a completed block inserted there
    done = int(w.positions()[reset_at]) // 64 - 1 if reset_at == 34 else -1
    S, N = rec["sel"][reset_at], rec["n_sel"][reset_at]
    inserted = np.array([[done in S[b, h, : N[b, h]] for h in range(w.n_kv_heads)] for b in range(w.batch)])
    assert np.array_equal(rec["n_miss"][reset_at], N - inserted)
    assert sum(int(m.sum()) for m in rec["n_miss"]) > sum(int(m.sum()) for m in base["n_miss"])
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            H.check_offload_unit(w, K, V, lam, q, rec, b, h, pool_reset_at=reset_at)
            _pool_consistent(layer, host, b, h)


@pytest.mark.parametrize("kq,ke,fused", [(8, 56, False), (32, 32, True), (64, 0, False)], ids=["kq8", "kq32", "kq64"])
def test_offload_sweep_points(kq, ke, fused):
    """The kq/k sweep points of the offload workload (k = 64, 16K context,
    pool of 80) at batch 2, every unit, 96 steps (one block completes); one
    of them with the gather folded into the attention."""
    _banner(f"offload sweep point kq={kq} ke={ke}: B=2, 16K context, pool 80, 96 steps, fused fetch {fused}")
    w = _w("offload", batch=2, n_steps=96, kq=kq, ke=ke)
    K, V, lam, q = NI.layer_inputs(w)
    rec, layer, host = H.run_offload(w, K, V, lam, q, fused_fetch=fused)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            H.check_offload_unit(w, K, V, lam, q, rec, b, h)
            _pool_consistent(layer, host, b, h)


# units whose attention outputs the full-size offload test compares (every
# unit's selections and pool tables are compared)
OFFLOAD_OUT_UNITS = ((0, 0), (9, 1), (17, 1), (26, 0), (40, 0), (45, 1), (58, 0), (63, 1))


@pytest.mark.parametrize("fused_fetch", [True, False], ids=["fused-fetch", "side-stream"])
def test_offload_workload_full_size(fused_fetch):
    """The offload workload at full size (B=64, 16K context, pool of 80, 128
    steps): the selections, miss lists, insert entries and physical slots of
    all 128 units, the pool contents of every unit against the host cache,
    and the outputs of eight units against the oracle."""
    _banner(f"offload workload: B=64, 16K context, pool 80, 128 steps (every unit), fused fetch {fused_fetch}")
    w = NI.WORKLOADS["offload"]
    K, V, lam, q = NI.layer_inputs(w)
    rec, layer, host = H.run_offload(w, K, V, lam, q, record_tables=False, fused_fetch=fused_fetch)
    misses = 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            st = H.check_offload_unit(w, K, V, lam, q, rec, b, h, outputs=(b, h) in OFFLOAD_OUT_UNITS)
            misses += st["misses"]
            _pool_consistent(layer, host, b, h)
    assert misses == sum(int(n.sum()) for n in rec["n_miss"])
    print(f"[offload] {misses} misses over {w.batch * w.n_kv_heads} units", flush=True)


def test_stack128k_full_size_layers():
    """Two layers of the 28-layer stack (the first and the last, with their
    own seeds) at full size: B=16, 131072-token context, pool of 80, 32 steps,
    run by the stack driver the bench times; every unit's selections and pool
    tables and three units' outputs of both layers against the oracle, every
    pool against the host caches."""
    _banner("stack128k: layers 0 and 27 at full size (B=16, 128K context, pool 80, 32 steps), every unit")
    w = NI.WORKLOADS["stack128k"]
    layer_ids = (0, w.n_layers - 1)
    positions = w.positions()
    blocks = [int(p) // 64 for p in positions]
    stack = R.OffloadStack(len(layer_ids), w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks,
                           w.dtype, w.kq, w.ke, w.pool_slots)
    inputs, qs = [], []
    for i, lid in enumerate(layer_ids):
        K, V, lam, q = NI.layer_inputs(w, lid, workers=NI.host_workers())
        stack.load_layer(i, K, V, lam, blocks[0], sorted(set(blocks)))
        inputs.append((K, V, lam, q))
        qs.append(torch.from_numpy(q).cuda().to(torch.bfloat16))
    pos = torch.from_numpy(np.repeat(positions[:, None], w.batch, axis=1).astype(np.int32)).cuda()
    keys = ("sel", "n_sel", "phys", "miss_list", "n_miss")
    rec = [{k: [] for k in keys + ("out",)} for _ in layer_ids]

    def on_layer(i, L):
        for k in keys:
            rec[i][k].append(getattr(L, k).clone())
        rec[i]["out"].append(L.out.float().clone())

    side = torch.cuda.Stream()
    for t in range(w.n_steps):
        stack.step(t, [qd[t] for qd in qs], pos[t], blocks[t], side, on_layer)
    torch.cuda.synchronize()
    for i, lid in enumerate(layer_ids):
        r = {k: [x.cpu().numpy() for x in v] for k, v in rec[i].items()}
        K, V, lam, q = inputs[i]
        misses = 0
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                st = H.check_offload_unit(w, K, V, lam, q, r, b, h, outputs=(b, h) in ((0, 0), (9, 1), (15, 1)))
                misses += st["misses"]
                _pool_consistent(stack.layers[i], stack.host[i], b, h)
        assert misses >= w.batch * w.n_kv_heads * (w.kq + w.ke), (lid, misses)     # at least the cold step's
        assert misses == sum(int(n.sum()) for n in r["n_miss"]), lid


@pytest.mark.parametrize("fused_fetch", [False, True], ids=["side-stream", "fused-fetch"])
def test_stack_small_crosses_blocks(fused_fetch):
    """The stack driver across block boundaries: three layers, a ragged
    prompt and 150 steps, so the window completes blocks that enter every
    layer's pool; every unit of every layer against the oracle."""
    _banner(f"stack: 3 layers, B=2, ragged prompt, 150 steps across blocks, pool 20, fused fetch {fused_fetch}")
    w = _w("stack128k", batch=2, prompt_len=64 * 30 + 41, n_steps=150, kq=6, ke=8, pool_slots=20, n_layers=3)
    positions = w.positions()
    blocks = [int(p) // 64 for p in positions]
    stack = R.OffloadStack(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype,
                           w.kq, w.ke, w.pool_slots)
    inputs, qs = [], []
    for l in range(w.n_layers):
        K, V, lam, q = NI.layer_inputs(w, l)
        stack.load_layer(l, K, V, lam, blocks[0], sorted(set(blocks)))
        inputs.append((K, V, lam, q))
        qs.append(torch.from_numpy(q).cuda().to(torch.bfloat16))
    pos = torch.from_numpy(np.repeat(positions[:, None], w.batch, axis=1).astype(np.int32)).cuda()
    keys = ("sel", "n_sel", "phys", "miss_list", "n_miss")
    rec = [{k: [] for k in keys + ("out",)} for _ in range(w.n_layers)]

    def on_layer(i, L):
        for k in keys:
            rec[i][k].append(getattr(L, k).clone())
        rec[i]["out"].append(L.out.float().clone())

    side = torch.cuda.Stream()
    for t in range(w.n_steps):
        stack.step(t, [qd[t] for qd in qs], pos[t], blocks[t], side, on_layer, fused_fetch=fused_fetch)
    torch.cuda.synchronize()
    assert blocks[-1] > blocks[0] + 1
    for l in range(w.n_layers):
        r = {k: [x.cpu().numpy() for x in v] for k, v in rec[l].items()}
        K, V, lam, q = inputs[l]
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                H.check_offload_unit(w, K, V, lam, q, r, b, h)
                _pool_consistent(stack.layers[l], stack.host[l], b, h)


@pytest.mark.parametrize("fused_fetch", [True, False], ids=["fused-fetch", "side-stream"])
def test_stack_ragged_positions(fused_fetch):
    """The stack driver with batch entries at their own positions (lags 0, 20
    and 45 tokens): per-entry window blocks, each entry's completed blocks
    pooled and inserted for that entry alone, in every layer; every unit of
    every layer against the oracle at its own positions."""
    _banner(f"stack: 3 layers, B=3, lags 0/20/45, 150 steps, pool 20, fused fetch {fused_fetch}")
    w = _w("stack128k", batch=3, prompt_len=64 * 30 + 41, n_steps=150, kq=6, ke=8, pool_slots=20, n_layers=3)
    lags = np.array([0, 20, 45])
    P = w.positions()[:, None] - lags[None, :]                       # [steps, B]
    C = P // 64
    stack = R.OffloadStack(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype,
                           w.kq, w.ke, w.pool_slots)
    inputs, qs = [], []
    for l in range(w.n_layers):
        K, V, lam, q = NI.layer_inputs(w, l)
        stack.load_layer(l, K, V, lam, C[0], sorted(set(C.ravel().tolist())))
        inputs.append((K, V, lam, q))
        qs.append(torch.from_numpy(q).cuda().to(torch.bfloat16))
    pos = torch.from_numpy(P.astype(np.int32)).cuda()
    keys = ("sel", "n_sel", "phys", "miss_list", "n_miss")
    rec = [{k: [] for k in keys + ("out",)} for _ in range(w.n_layers)]

    def on_layer(i, L):
        for k in keys:
            rec[i][k].append(getattr(L, k).clone())
        rec[i]["out"].append(L.out.float().clone())

    side = torch.cuda.Stream()
    for t in range(w.n_steps):
        stack.step(t, [qd[t] for qd in qs], pos[t], C[t], side, on_layer, fused_fetch=fused_fetch)
    torch.cuda.synchronize()
    steps_done = [set(np.nonzero(C[1:, b] > C[:-1, b])[0] + 1) for b in range(w.batch)]
    assert all(steps_done) and len(set().union(*steps_done)) == sum(map(len, steps_done))
    for l in range(w.n_layers):
        r = {k: [x.cpu().numpy() for x in v] for k, v in rec[l].items()}
        r["positions"] = P
        K, V, lam, q = inputs[l]
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                H.check_offload_unit(w, K, V, lam, q, r, b, h)
                _pool_consistent(stack.layers[l], stack.host[l], b, h)


def test_prefill128k_chunk_selection():
    _banner("prefill128k: pool 131072 tokens, select for 64 query rows")
    w = NI.WORKLOADS["prefill128k"]
    K, V, lam, q = NI.layer_inputs(w)                    # q: [64, 1, 16, 128]
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    layer = R.DecodeLayer(1, 16, 2, 128, w.n_blocks, "bf16", w.kq, w.ke)
    layer.pool_blocks(kv, logits, 0, w.n_blocks)
    n_q = w.n_steps
    qrows = qd.permute(1, 0, 2, 3).contiguous()           # [B, n_query, Hq, D]
    posr = pos.t().contiguous()                           # [B, n_query]
    sel = torch.full((1, n_q, 2, w.kq + w.ke), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((1, n_q, 2), dtype=torch.int32, device="cuda")
    ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, w.kq, w.ke), dtype=torch.uint8, device="cuda")
    nb.select_blocks(layer.dims, qrows, n_q, posr, layer.k_comp, layer.e_blk, w.kq, w.ke, sel, n_sel, ws)
    sel = sel.cpu().numpy()
    n_sel = n_sel.cpu().numpy()
    kc = layer.k_comp.float().cpu().numpy()
    for h in range(2):
        kbar = O.subblock_key_means(K[0, h], bf16=True)
        assert np.array_equal(kc[0, h].view(np.uint32), kbar.view(np.uint32))
        E = O.block_eviction_scores(O.subblock_logit_means(lam[0, h]))
        for r in range(n_q):
            p = int(w.positions()[r])
            c = p // 64
            s_q = O.query_block_scores(q[r, 0, h * 8:(h + 1) * 8], kbar, c)
            _, _, S = O.select_blocks(s_q, E, c, w.kq, w.ke)
            got = list(sel[0, r, h, : n_sel[0, r, h]])
            assert got == S or H.selection_ok(got, s_q, E, c, w.kq, w.ke), (h, r)


MULTI_CASES = [
    # name, workload overrides, n_query, kq, ke
    ("D128 G8", dict(), 13, 16, 48),
    ("D64 G4", dict(head_dim=64, n_q_heads=8), 21, 12, 20),
    ("D128 G1", dict(n_q_heads=2), 19, 8, 8),
    ("D64 G2 kq only", dict(head_dim=64, n_q_heads=4), 9, 30, 0),
]


@pytest.mark.parametrize("name,over,n_q,kq,ke", MULTI_CASES, ids=[c[0] for c in MULTI_CASES])
def test_select_many_rows_matches_oracle(name, over, n_q, kq, ke):
    """Chunks of query rows share one scan of the compressed keys; every row
    keeps its own window, including rows whose position is out of range."""
    _banner(f"select many rows {name}")
    T = 64 * 640 + 11
    w = _w("layer32k", batch=2, prompt_len=T, n_steps=1, kq=kq, ke=ke, prefill=True, **over)
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, kq, ke)
    layer.pool_blocks(kv, logits, 0, T // 64)
    rng = np.random.default_rng(5)
    qn = NI.round_to_bf16(rng.standard_normal((w.batch, n_q, w.n_q_heads, w.head_dim)).astype(np.float32))
    posn = rng.integers(0, T, size=(w.batch, n_q)).astype(np.int32)
    posn[0, 0], posn[1, n_q - 1], posn[0, n_q // 2] = -1, 64 * w.n_blocks + 5, 63
    qd = torch.from_numpy(qn).cuda().to(torch.bfloat16)
    posd = torch.from_numpy(posn).cuda()
    k_cap = kq + ke
    sel = torch.full((w.batch, n_q, w.n_kv_heads, k_cap), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((w.batch, n_q, w.n_kv_heads), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, kq, ke), dtype=torch.uint8, device="cuda")
    nb.select_blocks(layer.dims, qd, n_q, posd, layer.k_comp, layer.e_blk, kq, ke, sel, n_sel, ws)
    sel = sel.cpu().numpy()
    n_sel = n_sel.cpu().numpy()
    ties = 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            kbar = O.subblock_key_means(K[b, h], bf16=True)
            E = O.block_eviction_scores(O.subblock_logit_means(lam[b, h]))
            for r in range(n_q):
                p = int(posn[b, r])
                c = p // 64 if 0 <= p < 64 * w.n_blocks else 0
                s_q = O.query_block_scores(qn[b, r, h * w.group:(h + 1) * w.group], kbar, c)
                _, _, S = O.select_blocks(s_q, E, c, kq, ke)
                got = list(sel[b, r, h, : n_sel[b, r, h]])
                assert np.all(sel[b, r, h, n_sel[b, r, h]:] == -1), (b, r, h)
                if got != S:
                    assert H.selection_ok(got, s_q, E, c, kq, ke), (b, r, h, p, got, S)
                    ties += 1
    assert ties <= 2


SHARED_CASES = [
    # name, workload overrides, n_query, kq, ke, first row's position in batch entry 0 / 1
    ("D128 G8 64 rows", dict(), 64, 16, 48, (64 * 639, 64 * 500)),
    ("D64 G4 13 rows", dict(head_dim=64, n_q_heads=8), 13, 12, 20, (64 * 600 + 40, 64 * 3 + 1)),
    ("D128 G1 3 rows", dict(n_q_heads=2), 3, 8, 8, (64 * 100 + 7, 64 * 639 + 61)),
    ("D64 G2 1 row kq only", dict(head_dim=64, n_q_heads=4), 1, 30, 0, (64 * 200, 64 * 10)),
]


@pytest.mark.parametrize("name,over,n_q,kq,ke,starts", SHARED_CASES, ids=[c[0] for c in SHARED_CASES])
def test_select_shared_matches_oracle(name, over, n_q, kq, ke, starts):
    """One selection per (b, h) for all rows of a chunk (reading U20), written
    to every row, against the oracle; then each row's exact attention over it
    plus the row's own window."""
    _banner(f"chunk-shared selection {name}")
    _shared_case(64 * 640 + 11, over, n_q, kq, ke, starts, 23)


@pytest.mark.parametrize("seed", range(12))
def test_random_shared_selection_matches_oracle(seed):
    """Seeded random chunk-shared selections: head groupings 1-8, both head
    dims, 1 to 64 rows inside one block at a random offset of a ragged
    prompt, random budgets; the shared set against the oracle and every row's
    attention over it."""
    rng = np.random.default_rng(7000 + seed)
    G, hkv = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2]))
    T = int(rng.integers(300, 20000))
    T += 1 if T % 64 == 0 else 0
    kq, ke = int(rng.integers(0, 25)), int(rng.integers(0, 25))
    if kq + ke == 0:
        kq = 1
    n_q = int(rng.integers(1, 65))
    starts = []
    for _ in range(2):
        blk = int(rng.integers(1, T // 64))         # a block whose rows all lie inside the prompt
        lo = int(rng.integers(0, 64 - min(n_q, 64) + 1))
        starts.append(64 * blk + lo)
    over = dict(n_q_heads=G * hkv, n_kv_heads=hkv, head_dim=int(rng.choice([64, 128])))
    _banner(f"random chunk-shared selection {seed}: T {T} {over} rows {n_q} kq {kq} ke {ke} starts {starts}")
    _shared_case(T, over, n_q, kq, ke, tuple(starts), 8000 + seed)


def _shared_case(T, over, n_q, kq, ke, starts, seed):
    w = _w("layer32k", batch=2, prompt_len=T, n_steps=1, kq=kq, ke=ke, prefill=True, **over)
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, kq, ke)
    layer.pool_blocks(kv, logits, 0, T // 64)
    rng = np.random.default_rng(seed)
    qn = NI.round_to_bf16(rng.standard_normal((w.batch, n_q, w.n_q_heads, w.head_dim)).astype(np.float32))
    posn = np.stack([np.arange(n_q) + s for s in starts]).astype(np.int32)   # rows inside one block
    assert np.all(posn // 64 == posn[:, :1] // 64) and posn.max() < T
    qd = torch.from_numpy(qn).cuda().to(torch.bfloat16)
    posd = torch.from_numpy(posn).cuda()
    k_cap = kq + ke
    sel = torch.full((w.batch, n_q, w.n_kv_heads, k_cap), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((w.batch, n_q, w.n_kv_heads), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, kq, ke), dtype=torch.uint8, device="cuda")
    nb.select_blocks_shared(layer.dims, qd, n_q, posd, layer.k_comp, layer.e_blk, kq, ke, sel, n_sel, ws)
    out = torch.zeros((w.batch, n_q, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    wsa = torch.zeros(nb.workspace_size(layer.dims, nb.OP_ATTN, n_q, k_cap, 0), dtype=torch.uint8, device="cuda")
    nb.sparse_chunk_attn(layer.dims, qd, n_q, kv, sel, n_sel, k_cap, posd, None, out, wsa)
    sel = sel.cpu().numpy()
    n_sel = n_sel.cpu().numpy()
    out = out.float().cpu().numpy()
    G, D = w.group, w.head_dim
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            kbar = O.subblock_key_means(K[b, h], bf16=True)
            E = O.block_eviction_scores(O.subblock_logit_means(lam[b, h]))
            q_chunk = qn[b, :, h * G:(h + 1) * G]
            c = int(posn[b, 0]) // 64
            _, _, S = O.chunk_shared_selection(q_chunk, int(posn[b, 0]), kbar, E, kq, ke)
            got = list(sel[b, 0, h, : n_sel[b, 0, h]])
            for r in range(n_q):                        # the same set in every row, -1 after it
                assert n_sel[b, r, h] == len(got) and list(sel[b, r, h, : len(got)]) == got, (b, r, h)
                assert np.all(sel[b, r, h, len(got):] == -1), (b, r, h)
            if got != S:
                s_q = O.query_block_scores(q_chunk.reshape(-1, D), kbar, c)
                assert H.selection_ok(got, s_q, E, c, kq, ke), (b, h, got, S)
            for r in range(n_q):
                ref = O.round_output(O.sparse_attention(q_chunk[r], K[b, h], V[b, h], got, int(posn[b, r])),
                                     bf16=True)
                e = float(np.max(np.abs(out[b, r, h * G:(h + 1) * G] - ref)))
                assert e <= 2e-2, (b, r, h, e)


def test_chunk_selections_exact_ties():
    """Prefill-chunk selection (per-row MFMA scan, and the chunk-shared
    selection) on keys and eviction logits that repeat one of three block
    patterns: every score is shared by a third of the blocks, the budgets
    are filled by the lowest ids of a group of equal scores, and the sets
    must equal the oracle's exactly."""
    _banner("chunk selections with exact ties")
    T = 64 * 640 + 11
    w = _w("layer32k", batch=2, prompt_len=T, n_steps=1, prefill=True)
    K, V, lam, _ = NI.layer_inputs(w)
    rng = np.random.default_rng(31)
    pat = NI.round_to_bf16(rng.standard_normal((3, w.head_dim)).astype(np.float32))
    blk = np.arange(K.shape[2]) // 64
    K[:] = pat[blk % 3][None, None]
    lam[:] = np.float32([0.5, -1.0, 2.0])[(blk * 7 // 3) % 3][None, None]
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    layer.pool_blocks(kv, logits, 0, T // 64)
    n_q, k_cap, G = 13, w.kq + w.ke, w.group
    qn = NI.round_to_bf16(rng.standard_normal((w.batch, n_q, w.n_q_heads, w.head_dim)).astype(np.float32))
    qd = torch.from_numpy(qn).cuda().to(torch.bfloat16)
    kbar = [[O.subblock_key_means(K[b, h], bf16=True) for h in range(w.n_kv_heads)] for b in range(w.batch)]
    E = [[O.block_eviction_scores(O.subblock_logit_means(lam[b, h])) for h in range(w.n_kv_heads)]
         for b in range(w.batch)]

    def run(call, posn):
        sel = torch.full((w.batch, n_q, w.n_kv_heads, k_cap), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.full((w.batch, n_q, w.n_kv_heads), -7, dtype=torch.int32, device="cuda")
        ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, w.kq, w.ke), dtype=torch.uint8,
                         device="cuda")
        call(layer.dims, qd, n_q, torch.from_numpy(posn).cuda(), layer.k_comp, layer.e_blk, w.kq, w.ke, sel,
             n_sel, ws)
        return sel.cpu().numpy(), n_sel.cpu().numpy()

    posn = rng.integers(64 * 100, T, size=(w.batch, n_q)).astype(np.int32)
    sel, n_sel = run(nb.select_blocks, posn)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            for r in range(n_q):
                c = int(posn[b, r]) // 64
                s_q = O.query_block_scores(qn[b, r, h * G:(h + 1) * G], kbar[b][h], c)
                assert len(set(np.round(s_q[:c], 9))) == 3
                _, _, S = O.select_blocks(s_q, E[b][h], c, w.kq, w.ke)
                assert [int(x) for x in sel[b, r, h, : n_sel[b, r, h]]] == S, ("per-row", b, r, h)

    posn = np.stack([np.arange(n_q) + 64 * 600 + 3, np.arange(n_q) + 64 * 150 + 40]).astype(np.int32)
    sel, n_sel = run(nb.select_blocks_shared, posn)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            _, _, S = O.chunk_shared_selection(qn[b, :, h * G:(h + 1) * G], int(posn[b, 0]), kbar[b][h], E[b][h],
                                               w.kq, w.ke)
            for r in range(n_q):
                assert [int(x) for x in sel[b, r, h, : n_sel[b, r, h]]] == S, ("shared", b, r, h)


def _chunk_attention_case(w, K, V, lam, q_rows, pos_rows, kv, layer):
    """Select for the n_query rows, then attend each row over its own
    selection and causal window; every row of every KV head against the
    oracle's attention over the GPU's selection."""
    B, n_q = pos_rows.shape
    k_cap = w.kq + w.ke
    qd = torch.from_numpy(q_rows).cuda().to(torch.bfloat16)          # [B, n_q, Hq, D]
    posd = torch.from_numpy(pos_rows.astype(np.int32)).cuda()
    sel = torch.full((B, n_q, w.n_kv_heads, k_cap), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((B, n_q, w.n_kv_heads), dtype=torch.int32, device="cuda")
    ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, w.kq, w.ke), dtype=torch.uint8, device="cuda")
    nb.select_blocks(layer.dims, qd, n_q, posd, layer.k_comp, layer.e_blk, w.kq, w.ke, sel, n_sel, ws)
    # a sentinel, so rows the call fails to write (zeros for rows out of range) show
    out = torch.full((B, n_q, w.n_q_heads, w.head_dim), 3.0, dtype=torch.bfloat16, device="cuda")
    wsa = torch.zeros(nb.workspace_size(layer.dims, nb.OP_ATTN, n_q, k_cap, 0), dtype=torch.uint8, device="cuda")
    nb.sparse_chunk_attn(layer.dims, qd, n_q, kv, sel, n_sel, k_cap, posd, None, out, wsa)
    sel = sel.cpu().numpy()
    n_sel = n_sel.cpu().numpy()
    out = out.float().cpu().numpy()
    G = w.group
    err = 0.0
    for b in range(B):
        for r in range(n_q):
            p = int(pos_rows[b, r])
            for h in range(w.n_kv_heads):
                S = list(sel[b, r, h, : n_sel[b, r, h]])
                if not 0 <= p < 64 * w.n_blocks:
                    assert np.all(out[b, r, h * G:(h + 1) * G] == 0.0)
                    continue
                ref = O.round_output(O.sparse_attention(q_rows[b, r, h * G:(h + 1) * G], K[b, h], V[b, h], S, p),
                                     bf16=True)
                e = float(np.max(np.abs(out[b, r, h * G:(h + 1) * G] - ref)))
                assert e <= 2e-2, (b, r, h, e)
                err = max(err, e)
    return err


def _random_prefill_config(seed):
    """A small seeded prefill configuration: heads, dtype, a ragged prompt,
    the number of query rows and the budgets."""
    rng = np.random.default_rng(3000 + seed)
    G, hkv = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2]))
    T = int(rng.integers(200, 20000))
    T += 1 if T % 64 == 0 else 0
    kq, ke = int(rng.integers(0, 25)), int(rng.integers(0, 25))
    if kq + ke == 0:
        kq = 1
    over = dict(batch=int(rng.integers(1, 4)), n_q_heads=G * hkv, n_kv_heads=hkv,
                head_dim=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])), prompt_len=T,
                n_steps=1, kq=kq, ke=ke, prefill=True)
    return over, int(rng.integers(1, 41))


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill_configs_match_oracle(seed):
    """Seeded random prefill chunks: query rows at scattered positions of a
    ragged prompt (a few out of range on either side), selected by
    nosa_select_blocks (the row-chunk MFMA scan from 8 rows on, bf16) and
    attended by nosa_sparse_chunk_attn (packed rows for bf16 with 4 or 8
    heads per KV head, one row per unit otherwise); every row's set against
    the oracle's top-k and its output against the oracle's attention over it."""
    over, n_q = _random_prefill_config(seed)
    _banner(f"random prefill {seed}: {over}, {n_q} rows")
    w = _w("layer32k", **over)
    T, bf16, G, k_cap = w.prompt_len, w.dtype == "bf16", w.group, w.kq + w.ke
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    layer.pool_blocks(kv, logits, 0, T // 64)
    rng = np.random.default_rng(4000 + seed)
    qn = rng.standard_normal((w.batch, n_q, w.n_q_heads, w.head_dim)).astype(np.float32)
    qn = NI.round_to_bf16(qn) if bf16 else qn
    posn = rng.integers(0, T, size=(w.batch, n_q)).astype(np.int32)
    odd = rng.random((w.batch, n_q))
    posn[odd < 0.08] = -1
    posn[odd > 0.94] = 64 * w.n_blocks + 3
    tdt = torch.bfloat16 if bf16 else torch.float32
    qd = torch.from_numpy(qn).cuda().to(tdt)
    posd = torch.from_numpy(posn).cuda()
    sel = torch.full((w.batch, n_q, w.n_kv_heads, k_cap), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((w.batch, n_q, w.n_kv_heads), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, w.kq, w.ke), dtype=torch.uint8, device="cuda")
    nb.select_blocks(layer.dims, qd, n_q, posd, layer.k_comp, layer.e_blk, w.kq, w.ke, sel, n_sel, ws)
    out = torch.full((w.batch, n_q, w.n_q_heads, w.head_dim), 3.0, dtype=tdt, device="cuda")
    wsa = torch.zeros(nb.workspace_size(layer.dims, nb.OP_ATTN, n_q, k_cap, 0), dtype=torch.uint8, device="cuda")
    nb.sparse_chunk_attn(layer.dims, qd, n_q, kv, sel, n_sel, k_cap, posd, None, out, wsa)
    sel, n_sel, out = sel.cpu().numpy(), n_sel.cpu().numpy(), out.float().cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            kbar = O.subblock_key_means(K[b, h], bf16=bf16)
            E = O.block_eviction_scores(O.subblock_logit_means(lam[b, h]))
            for r in range(n_q):
                p = int(posn[b, r])
                rows = out[b, r, h * G:(h + 1) * G]
                got = [int(x) for x in sel[b, r, h, : n_sel[b, r, h]]]
                assert np.all(sel[b, r, h, n_sel[b, r, h]:] == -1), (b, r, h)
                if not 0 <= p < 64 * w.n_blocks:
                    assert got == [] and np.all(rows == 0.0), (b, r, h, p)
                    continue
                c = p // 64
                s_q = O.query_block_scores(qn[b, r, h * G:(h + 1) * G], kbar, c)
                _, _, S = O.select_blocks(s_q, E, c, w.kq, w.ke)
                if got != S:
                    assert H.selection_ok(got, s_q, E, c, w.kq, w.ke), (b, r, h, p, got, S)
                ref = O.round_output(O.sparse_attention(qn[b, r, h * G:(h + 1) * G], K[b, h], V[b, h], got, p),
                                     bf16=bf16)
                e = float(np.max(np.abs(rows - ref)))
                assert e <= H.ATOL[w.dtype], (b, r, h, p, e)


def test_chunk_attention_small():
    """Ragged prompt, two batch entries, 21 rows at scattered positions (five
    out of range, four of them a whole packed group), G = 4, D = 64."""
    _banner("chunk attention: B=2, 21 rows, D64 G4")
    T = 64 * 90 + 13
    w = _w("layer32k", batch=2, prompt_len=T, n_steps=1, head_dim=64, n_q_heads=8, kq=10, ke=14, prefill=True)
    K, V, lam, _ = NI.layer_inputs(w)
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, np.zeros((1, 1, 1, 1), np.float32))
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    layer.pool_blocks(kv, logits, 0, T // 64)
    rng = np.random.default_rng(17)
    q_rows = NI.round_to_bf16(rng.standard_normal((w.batch, 21, w.n_q_heads, w.head_dim)).astype(np.float32))
    pos_rows = rng.integers(0, T, size=(w.batch, 21))
    pos_rows[1, 3] = -1
    pos_rows[1, 4:8] = -1          # a whole group of four rows (G = 4 packs four rows per MFMA tile)
    pos_rows[0, 5] = 63
    _chunk_attention_case(w, K, V, lam, q_rows, pos_rows, kv, layer)


def test_prefill128k_chunk_attention():
    """The prefill128k workload at full size: 64 query rows at the end of the
    131072-token prompt, each over its own selection and window."""
    _banner("prefill128k: selection and attention for 64 query rows")
    w = NI.WORKLOADS["prefill128k"]
    K, V, lam, q = NI.layer_inputs(w)                                # q: [64, 1, 16, 128]
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, q)
    layer = R.DecodeLayer(1, 16, 2, 128, w.n_blocks, "bf16", w.kq, w.ke)
    layer.pool_blocks(kv, logits, 0, w.n_blocks)
    q_rows = np.ascontiguousarray(q.transpose(1, 0, 2, 3))           # [B, n_query, Hq, D]
    pos_rows = w.positions()[None, :].astype(np.int64)
    _chunk_attention_case(w, K, V, lam, q_rows, pos_rows, kv, layer)


def test_prefill128k_shared_selection():
    """prefill128k at full size: one shared selection for the 64 rows at the
    end of the 131072-token prompt (block 2047), and their attention over it;
    every selection and a sample of rows against the oracle."""
    _banner("prefill128k: chunk-shared selection and attention, 64 rows")
    w = NI.WORKLOADS["prefill128k"]
    K, V, lam, q = NI.layer_inputs(w)                                # q: [64, 1, 16, 128]
    kv, logits, _, _ = H.device_inputs(w, K, V, lam, q)
    layer = R.DecodeLayer(1, 16, 2, 128, w.n_blocks, "bf16", w.kq, w.ke)
    layer.pool_blocks(kv, logits, 0, w.n_blocks)
    q_rows = np.ascontiguousarray(q.transpose(1, 0, 2, 3))           # [1, 64, 16, 128]
    pos_rows = w.positions()[None, :].astype(np.int32)
    n_q, k_cap = pos_rows.shape[1], w.kq + w.ke
    qd = torch.from_numpy(q_rows).cuda().to(torch.bfloat16)
    posd = torch.from_numpy(pos_rows).cuda()
    sel = torch.full((1, n_q, 2, k_cap), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((1, n_q, 2), dtype=torch.int32, device="cuda")
    ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, w.kq, w.ke), dtype=torch.uint8, device="cuda")
    nb.select_blocks_shared(layer.dims, qd, n_q, posd, layer.k_comp, layer.e_blk, w.kq, w.ke, sel, n_sel, ws)
    out = torch.zeros((1, n_q, 16, 128), dtype=torch.bfloat16, device="cuda")
    wsa = torch.zeros(nb.workspace_size(layer.dims, nb.OP_ATTN, n_q, k_cap, 0), dtype=torch.uint8, device="cuda")
    nb.sparse_chunk_attn(layer.dims, qd, n_q, kv, sel, n_sel, k_cap, posd, None, out, wsa)
    sel = sel.cpu().numpy()
    n_sel = n_sel.cpu().numpy()
    out = out.float().cpu().numpy()
    c = int(pos_rows[0, 0]) // 64
    for h in range(2):
        kbar = O.subblock_key_means(K[0, h], bf16=True)
        E = O.block_eviction_scores(O.subblock_logit_means(lam[0, h]))
        q_chunk = q_rows[0, :, h * 8:(h + 1) * 8]
        _, _, S = O.chunk_shared_selection(q_chunk, int(pos_rows[0, 0]), kbar, E, w.kq, w.ke)
        got = list(sel[0, 0, h, : n_sel[0, 0, h]])
        assert all(list(sel[0, r, h, : n_sel[0, r, h]]) == got for r in range(n_q))
        if got != S:
            s_q = O.query_block_scores(q_chunk.reshape(-1, 128), kbar, c)
            assert H.selection_ok(got, s_q, E, c, w.kq, w.ke), (h, got, S)
        for r in (0, 1, 31, 62, 63):
            ref = O.round_output(O.sparse_attention(q_chunk[r], K[0, h], V[0, h], got, int(pos_rows[0, r])),
                                 bf16=True)
            assert float(np.max(np.abs(out[0, r, h * 8:(h + 1) * 8] - ref))) <= 2e-2, (h, r)


SPLIT_CASES = [
    # name, dtype, D, Hq, Hkv, d_e, B, n_tok, contiguous positions
    ("bf16 D128 G8 decode", "bf16", 128, 16, 2, 128, 8, 1, False),
    ("bf16 D64 G4 chunk", "bf16", 64, 8, 2, 48, 2, 70, False),
    ("f32 D64 G2", "f32", 64, 4, 2, 96, 3, 9, False),
    ("f32 D128 G4 chunk", "f32", 128, 8, 2, 80, 2, 37, False),
    ("bf16 D128 G8 prefill chunk", "bf16", 128, 16, 2, 128, 2, 300, True),
]


@pytest.mark.parametrize("name,dtype,D,Hq,Hkv,d_e,B,n_tok,contig", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_qkv_matches_oracle(name, dtype, D, Hq, Hkv, d_e, B, n_tok, contig):
    """q copied, k and v written into the cache's block format at their
    positions (bit-exact against packing the same rows), eviction logits
    against the oracle's Eq. 4 in float64.  Chunks of 16 or more tokens take
    the 16-tokens-per-workgroup path (ragged last group included)."""
    _banner(f"split qkv {name}")
    _split_qkv_case(dtype, D, Hq, Hkv, d_e, B, n_tok, contig, 21)


@pytest.mark.parametrize("seed", range(16))
def test_random_split_qkv_matches_oracle(seed):
    """Seeded random QKV splits: head groupings 1-8, 1 to 4 KV heads, both
    head dims and dtypes, eviction hidden sizes 1 to 300, 1 to 100 tokens at
    scattered or consecutive positions."""
    rng = np.random.default_rng(5000 + seed)
    G, Hkv, D = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 4])), int(rng.choice([64, 128]))
    case = (str(rng.choice(["bf16", "f32"])), D, G * Hkv, Hkv, int(rng.integers(1, 301)), int(rng.integers(1, 5)),
            int(rng.integers(1, 101)), bool(rng.random() < 0.4))
    _banner(f"random split qkv {seed}: {case}")
    _split_qkv_case(*case, 6000 + seed)


def _split_qkv_case(dtype, D, Hq, Hkv, d_e, B, n_tok, contig, seed):
    NB = 12
    rng = np.random.default_rng(seed)
    row = (Hq + 2 * Hkv) * D
    qkv = rng.standard_normal((B, n_tok, row)).astype(np.float32)
    if dtype == "bf16":
        qkv = NI.round_to_bf16(qkv)
    if contig:      # a prefill chunk: consecutive positions from an unaligned start
        pos = np.stack([np.arange(n_tok) + 5 + 64 * b for b in range(B)]).astype(np.int32)
    else:
        pos = np.stack([rng.permutation(NB * 64)[:n_tok] for _ in range(B)]).astype(np.int32)
    if n_tok > 2:
        pos[0, 1] = -1
        pos[B - 1, 2] = NB * 64 + 3
    w1 = (rng.standard_normal((Hkv, D, d_e)) / math.sqrt(D)).astype(np.float32)
    w2 = rng.standard_normal((Hkv, d_e)).astype(np.float32)
    tdt = R.torch_dtype(dtype)
    d = nb.dims(B, Hq, Hkv, D, NB, dtype)
    q_out = torch.zeros((B, n_tok, Hq, D), dtype=tdt, device="cuda")
    kv = torch.zeros((B, Hkv, NB, 2 * 64 * D), dtype=tdt, device="cuda")
    lg = torch.zeros((B, Hkv, NB * 64), dtype=torch.float32, device="cuda")
    nb.split_qkv(d, torch.from_numpy(qkv).cuda().to(tdt), n_tok, torch.from_numpy(pos).cuda(),
                 torch.from_numpy(w1).cuda(), torch.from_numpy(w2).cuda(), d_e, q_out, kv, lg)
    torch.cuda.synchronize()
    assert np.array_equal(q_out.float().cpu().numpy().reshape(B, n_tok, Hq * D), qkv[:, :, : Hq * D])
    K = np.zeros((B, Hkv, NB * 64, D), np.float32)
    V = np.zeros_like(K)
    ref_lg = np.zeros((B, Hkv, NB * 64), np.float64)
    for b in range(B):
        for t in range(n_tok):
            p = int(pos[b, t])
            if not 0 <= p < NB * 64:
                continue
            for h in range(Hkv):
                K[b, h, p] = qkv[b, t, (Hq + h) * D:(Hq + h + 1) * D]
                V[b, h, p] = qkv[b, t, (Hq + Hkv + h) * D:(Hq + Hkv + h + 1) * D]
                ref_lg[b, h, p] = O.eviction_logits(V[b, h, p][None, :], w1[h], w2[h])[0]
    want = R.to_device_blocks(K, V, NB, dtype)
    assert torch.equal(kv.view(torch.int16) if dtype == "bf16" else kv, want.view(torch.int16) if dtype == "bf16" else want)
    got = lg.cpu().numpy()
    scale = np.abs(w2).sum() * 4.0
    assert np.max(np.abs(got - ref_lg)) <= 1e-5 * scale


# ---------------------------------------------------- one-launch decode step
@pytest.mark.parametrize("wname,over", [
    ("tiny", {}),
    ("layer32k", dict(batch=3, prompt_len=64 * 40 + 50, n_steps=100)),     # crosses block ends
    ("layer32k", dict(batch=2, prompt_len=64 * 200 + 7, n_steps=70, kq=5, ke=0)),
    ("layer32k", dict(batch=2, prompt_len=64 * 30 + 60, n_steps=10, kq=0, ke=9, head_dim=64, n_q_heads=4)),
    ("layer32k", dict(batch=2, prompt_len=64 * 10 + 5, n_steps=70)),          # fewer candidates than kq
    ("layer32k", dict(batch=2, prompt_len=5, n_steps=70)),                    # no candidates, then one
], ids=["tiny", "boundaries", "kq-only", "ke-only-D64", "short-context", "first-block"])
def test_fused_step_matches_oracle(wname, over):
    _banner(f"fused step {wname} {over}")
    w = NI.scaled(NI.WORKLOADS[wname], **over) if over else NI.WORKLOADS[wname]
    K, V, lam, q = NI.layer_inputs(w)
    s1, n1, o1, layer = H.run_resident(w, K, V, lam, q, fused=True)
    assert layer.step_timeouts() == 0
    s2, n2, o2, _ = H.run_resident(w, K, V, lam, q, fused=False)
    for a, b in zip(n1, n2):
        assert np.array_equal(a, b)
    for a, b in zip(s1, s2):
        assert np.array_equal(a, b)            # same scan arithmetic: identical sets
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            H.compare_unit(w, K, V, lam, q, b, h, H.unit_selections(s1, n1, b, h), gpu_out=o1)


def _random_config(seed):
    """A small seeded configuration: head grouping, head dim, dtype, batch,
    ragged prompt length (never a multiple of 64), budgets, step count."""
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    L = int(rng.integers(65, 6000))
    L += 1 if L % 64 == 0 else 0
    kq, ke = int(rng.integers(0, 25)), int(rng.integers(0, 25))
    if kq + ke == 0:
        kq = 1
    return dict(batch=int(rng.integers(1, 6)), n_q_heads=G * hkv, n_kv_heads=hkv,
                head_dim=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])), prompt_len=L,
                n_steps=int(rng.integers(3, 41)), kq=kq, ke=ke)


@pytest.mark.parametrize("seed", range(32))
def test_random_configs_match_oracle(seed):
    """Seeded random shapes through both resident paths (the one-launch step
    and the separate calls), every unit against the oracle: head groupings 1,
    2, 4 and 8, head dims 64 and 128, both dtypes, budgets from 0 to 24,
    prompts up to 6000 tokens and up to 40 steps (so some cross block ends)."""
    over = _random_config(seed)
    _banner(f"random config {seed}: {over}")
    w = NI.scaled(NI.WORKLOADS["layer32k"], **over)
    K, V, lam, q = NI.layer_inputs(w)
    s1, n1, o1, layer = H.run_resident(w, K, V, lam, q, fused=True)
    assert layer.step_timeouts() == 0
    s2, n2, o2, _ = H.run_resident(w, K, V, lam, q, fused=False)
    for a, b in zip(n1, n2):
        assert np.array_equal(a, b)
    for a, b in zip(s1, s2):
        assert np.array_equal(a, b)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            H.compare_unit(w, K, V, lam, q, b, h, H.unit_selections(s1, n1, b, h), gpu_out=o1)
            H.compare_unit(w, K, V, lam, q, b, h, H.unit_selections(s2, n2, b, h), gpu_out=o2)


@pytest.mark.parametrize("fused", [True, False], ids=["one-launch", "separate-calls"])
def test_exact_ties_break_by_block_id(fused):
    """Blocks whose keys and eviction logits repeat one of three patterns
    score exactly alike (the same arithmetic on the same values), so each
    budget is filled from a group of equal scores; Eq. 7's top-k then
    keeps the lowest ids of that group (score desc, id asc) on both sides,
    and the sets must equal the oracle's exactly, with no tie allowance."""
    _banner(f"exact ties, fused={fused}")
    w = NI.scaled(NI.WORKLOADS["layer32k"], batch=2, prompt_len=64 * 60 + 40, n_steps=40)
    K, V, lam, q = NI.layer_inputs(w)
    rng = np.random.default_rng(7)
    pat = torch.from_numpy(rng.standard_normal((3, w.head_dim)).astype(np.float32))
    pat = pat.to(torch.bfloat16).float().numpy()
    blk = np.arange(K.shape[2]) // 64
    K[:] = pat[blk % 3][None, None]
    lam[:] = np.float32([0.5, -1.0, 2.0])[(blk * 7 // 3) % 3][None, None]
    s1, n1, o1, layer = H.run_resident(w, K, V, lam, q, fused=fused)
    if fused:
        assert layer.step_timeouts() == 0
    positions = w.positions()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            sel = H.unit_selections(s1, n1, b, h)
            tr, _ = H.oracle_scores(w, K, V, lam, q, b, h)
            for t, S in enumerate(sel):
                c = int(positions[t]) // 64
                assert len(set(np.round(tr.s_q[t][:c], 12))) == 3      # three distinct scores, many blocks each
                assert [int(x) for x in S] == tr.sel[t], f"unit ({b},{h}) step {t}"
            st = H.compare_unit(w, K, V, lam, q, b, h, sel, gpu_out=o1)
            assert st["ties"] == 0


def test_fused_step_layer32k_full():
    _banner("fused step on the full layer32k workload")
    w = NI.WORKLOADS["layer32k"]
    K, V, lam, q = NI.layer_inputs(w)
    s1, n1, o1, layer = H.run_resident(w, K, V, lam, q, fused=True)
    assert layer.step_timeouts() == 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            H.compare_unit(w, K, V, lam, q, b, h, H.unit_selections(s1, n1, b, h), gpu_out=o1)


def test_max_size_context_and_budget():
    """The largest configuration the calls accept: 4096 blocks (a 256K-token
    context) and k = 256 blocks (kq 64 + ke 192), the last steps of the
    cache; the one-launch step against the separate calls (identical sets)
    and against the oracle for every unit and step."""
    _banner("max size: 4096 blocks, k = 256")
    w = NI.scaled(NI.WORKLOADS["layer32k"], batch=1, prompt_len=64 * 4096 - 10, n_steps=5, kq=64, ke=192)
    assert w.n_blocks == 4096
    K, V, lam, q = NI.layer_inputs(w)
    s1, n1, o1, layer = H.run_resident(w, K, V, lam, q, fused=True)
    assert layer.step_timeouts() == 0
    s2, n2, o2, _ = H.run_resident(w, K, V, lam, q, fused=False)
    for a, b in zip(n1, n2):
        assert np.array_equal(a, b)
    for a, b in zip(s1, s2):
        assert np.array_equal(a, b)
    assert all(int(n.max()) > 200 for n in n1)        # kq + ke minus the overlap of the two top-k sets
    for h in range(w.n_kv_heads):
        H.compare_unit(w, K, V, lam, q, 0, h, H.unit_selections(s1, n1, 0, h), gpu_out=o1)


def test_expired_score_waits_are_counted_and_poison_outputs():
    """Failure handling of the one-launch step, forced from the host (the
    library's test hook): every query-aware worker's score wait runs to a
    short bound.  The launch must count the expired waits and write NaN for
    every output, and every kernel must still finish.  With the hook off the
    same workspace runs the next step exactly (against the separate calls)
    and counts nothing more."""
    _banner("expired score waits (host-forced)")
    w = NI.scaled(NI.WORKLOADS["layer32k"], batch=2, prompt_len=64 * 40 + 10, n_steps=2)
    K, V, lam, q = NI.layer_inputs(w)
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    c0 = int(w.positions()[0]) // 64
    layers = []
    for _ in range(2):
        L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
        L.pool_blocks(kv, logits, 0, c0)
        layers.append(L)
    fused, ref = layers
    nb.debug_expire_step_waits(True)
    try:
        fused.step_fused(qd[0], kv, pos[0])
        torch.cuda.synchronize()
        bad = fused.out.float().cpu().numpy()
    finally:
        nb.debug_expire_step_waits(False)
    n_bad = fused.step_timeouts()
    assert n_bad > 0
    assert np.all(np.isnan(bad))
    fused.step_fused(qd[1], kv, pos[1])
    ref.step_resident(qd[1], kv, pos[1])
    torch.cuda.synchronize()
    assert fused.step_timeouts() == n_bad
    assert np.array_equal(fused.n_sel.cpu().numpy(), ref.n_sel.cpu().numpy())
    assert np.array_equal(fused.sel.cpu().numpy(), ref.sel.cpu().numpy())
    out = fused.out.float().cpu().numpy()
    assert np.all(np.isfinite(out))
    assert float(np.max(np.abs(out - ref.out.float().cpu().numpy()))) < 2e-2


@pytest.mark.parametrize("batch", [32, 64], ids=["64-units", "128-units"])
def test_fused_step_many_units(batch):
    """Many (b, h) units: few workgroups per unit (a single E worker scanning
    in several rounds, several halves per wavefront) and, at 128 units, more
    workgroups than CUs, so later ones start only as earlier ones finish."""
    _banner(f"fused step with {2 * batch} units")
    w = NI.scaled(NI.WORKLOADS["layer32k"], batch=batch, prompt_len=64 * 100 + 10, n_steps=5)
    K, V, lam, q = NI.layer_inputs(w)
    s1, n1, o1, layer = H.run_resident(w, K, V, lam, q, fused=True)
    assert layer.step_timeouts() == 0
    s2, n2, o2, _ = H.run_resident(w, K, V, lam, q, fused=False)
    for a, b in zip(n1, n2):
        assert np.array_equal(a, b)
    for a, b in zip(s1, s2):
        assert np.array_equal(a, b)
    for a, b in zip(o1, o2):
        assert float(np.max(np.abs(a - b))) < 2e-2
    for b in (0, batch - 1):
        for h in range(w.n_kv_heads):
            H.compare_unit(w, K, V, lam, q, b, h, H.unit_selections(s1, n1, b, h), gpu_out=o1)
