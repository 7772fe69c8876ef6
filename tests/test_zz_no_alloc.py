"""nosa_decode_step_static (the one-launch step on the library's own
workspace, for callers that cannot allocate) against nosa_decode_step with a
caller workspace, through the C ABI: identical selections, outputs within the
bf16 bar, on consecutive calls whose geometry changes (the second input is
smaller), and on two layers sharing the static workspace."""
import numpy as np
import pytest
import torch

import nosa_inputs as NI
from kv_cache_offload_amd import binding as nb
from kv_cache_offload_amd import runner as R
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nb.load()
    yield
    torch.cuda.synchronize()


def _layer(w, seed_shift=0):
    K, V, lam, q = NI.layer_inputs(w)
    if seed_shift:
        lam = np.roll(lam, seed_shift * 64, axis=2)       # another layer: other eviction scores
    kv, logits, qd, pos = H.device_inputs(w, K, V, lam, q)
    L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    L.pool_blocks(kv, logits, 0, int(w.positions()[0]) // 64)
    return dict(w=w, K=K, V=V, lam=lam, q=q, kv=kv, qd=qd, pos=pos, layer=L)


def _both(case, t):
    """Step t through nosa_decode_step (caller workspace) and through
    nosa_decode_step_static; returns (sel, n_sel, out) of each."""
    w, L = case["w"], case["layer"]
    print(f"[case] static step B={w.batch} NB={w.n_blocks} kq={w.kq} ke={w.ke} t={t}", flush=True)
    L.step_fused(case["qd"][t], case["kv"], case["pos"][t])
    ref = (L.sel.clone(), L.n_sel.clone(), L.out.float().clone())
    sel = torch.full_like(L.sel, -7)
    n_sel = torch.full_like(L.n_sel, -7)
    out = torch.full_like(L.out, float("nan"))
    nb.decode_step_static(L.dims, case["qd"][t], case["pos"][t], L.k_comp, L.e_blk, w.kq, w.ke, case["kv"],
                          L.scale, sel, n_sel, out)
    torch.cuda.synchronize()
    return ref, (sel, n_sel, out.float())


def _check(case, t, ref, got):
    (s0, n0, o0), (s1, n1, o1) = ref, got
    assert torch.equal(n0, n1)
    assert torch.equal(s0, s1)
    err = float((o0 - o1).abs().max())
    assert err <= H.ATOL[case["w"].dtype], err
    # and the static step against the oracle, unit by unit
    w = case["w"]
    S, N, O = s1.cpu().numpy(), n1.cpu().numpy(), o1.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            sel = [list(S[b, h, : N[b, h]])]
            one = NI.scaled(w, n_steps=1, prompt_len=int(w.positions()[t]))
            H.compare_unit(one, case["K"], case["V"], case["lam"], case["q"][t:t + 1], b, h, sel, gpu_out=[O])


def test_static_step_matches_workspace_step():
    big = _layer(NI.scaled(NI.WORKLOADS["layer32k"], batch=4, prompt_len=64 * 150 + 20, n_steps=3))
    small = _layer(NI.scaled(NI.WORKLOADS["layer32k"], batch=2, prompt_len=64 * 60 + 3, n_steps=2, kq=8, ke=24))
    # two calls in a row, the second with a smaller input (another geometry:
    # the static workspace is cleared in between)
    ref, got = _both(big, 0)
    _check(big, 0, ref, got)
    ref, got = _both(small, 0)
    _check(small, 0, ref, got)
    # back to the first geometry, then consecutive steps of one geometry
    for t in (1, 2):
        ref, got = _both(big, t)
        _check(big, t, ref, got)
    # a second layer of the same geometry shares the static workspace: its
    # own eviction scores give its own Gamma_e (the cache is keyed by address)
    other = _layer(NI.scaled(NI.WORKLOADS["layer32k"], batch=4, prompt_len=64 * 150 + 20, n_steps=3), seed_shift=5)
    for case in (other, big, other):
        ref, got = _both(case, 1)
        _check(case, 1, ref, got)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = big["layer"]
    nb.step_timeouts(L.dims, L.kq, L.ke, None, out)
    assert int(out.item()) == 0


def test_static_step_replayed_from_a_graph():
    """Callers under graph capture: three static steps captured in one graph
    (their geometry's first call made before the capture, so the graph holds
    the step launches only) and replayed four times, with buffer fills and an
    eager static step of the same geometry between the replays: every replay
    gives the eager calls' selections and outputs bit for bit, and no wait
    expires."""
    case = _layer(NI.scaled(NI.WORKLOADS["layer32k"], batch=4, prompt_len=64 * 150 + 20, n_steps=3))
    w, L = case["w"], case["layer"]
    eager = [_both(case, t)[1] for t in range(w.n_steps)]
    bufs = [(torch.empty_like(L.sel), torch.empty_like(L.n_sel), torch.empty_like(L.out)) for _ in range(w.n_steps)]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for t, (sel, n_sel, out) in enumerate(bufs):
            nb.decode_step_static(L.dims, case["qd"][t], case["pos"][t], L.k_comp, L.e_blk, w.kq, w.ke, case["kv"],
                                  L.scale, sel, n_sel, out)
    for rep in range(4):
        print(f"[case] static step graph replay {rep}", flush=True)
        for sel, n_sel, out in bufs:
            sel.fill_(-7)
            n_sel.fill_(-7)
            out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t, (sel, n_sel, out) in enumerate(bufs):
            s0, n0, o0 = eager[t]
            assert torch.equal(n_sel, n0) and torch.equal(sel, s0), f"replay {rep}, step {t}: selection"
            assert torch.equal(out.float(), o0), f"replay {rep}, step {t}: output"
        _both(case, rep % w.n_steps)      # an eager static step between the replays
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    nb.step_timeouts(L.dims, L.kq, L.ke, None, out)
    assert int(out.item()) == 0
