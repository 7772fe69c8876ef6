"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle on the same seeded inputs."""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np
import torch

import nosa_inputs as NI
from kv_cache_offload_amd import runner as R
from oracle import nosa_oracle as O

REL_TIE = 1e-5            # score window inside which either order is accepted
ATOL = {"bf16": 2e-2, "f32": 1e-4}


def selection_ok(S_gpu, s_q, E, c, kq, ke, rel=REL_TIE) -> bool:
    """S_gpu is Gamma_q' U Gamma_e where Gamma_e is the exact top-ke of E and
    Gamma_q' is a top-kq set of s_q once scores within `rel` of the kq-th
    best are treated as equal."""
    S = set(int(x) for x in S_gpu)
    g_e = set(O.top_blocks(list(E[:c]), ke))
    if not g_e <= S or any(j < 0 or j >= c for j in S):
        return False
    kk = min(kq, c)
    if kk == 0:
        return S == g_e
    order = O.top_blocks(list(s_q[:c]), c)
    thr = float(s_q[order[kk - 1]])
    tie = {j for j in range(c) if abs(float(s_q[j]) - thr) <= rel * max(abs(float(s_q[j])), abs(thr))}
    must = {j for j in range(c) if float(s_q[j]) > thr and j not in tie}
    qpart = S - g_e
    if not qpart <= (must | tie) or not must <= S:
        return False
    base = must | qpart
    extra = (tie & g_e) - base
    return len(base) <= kk <= len(base) + len(extra)


def device_inputs(w: NI.Workload, K, V, lam, q, device="cuda"):
    NB = w.n_blocks
    kv = R.to_device_blocks(K, V, NB, w.dtype, device)
    logits = R.pad_logits(torch.from_numpy(lam).to(device), NB)
    qd = torch.from_numpy(q).to(device=device, dtype=R.torch_dtype(w.dtype))     # [n, B, Hq, D]
    pos = torch.from_numpy(np.repeat(w.positions()[:, None], w.batch, axis=1).astype(np.int32)).to(device)
    return kv, logits, qd, pos


def run_resident(w: NI.Workload, K, V, lam, q, steps: Optional[int] = None, fused: bool = False):
    """GPU decode in resident mode (separate calls, or the one-launch step);
    returns per-step sel lists and outputs."""
    n = w.n_steps if steps is None else steps
    kv, logits, qd, pos = device_inputs(w, K, V, lam, q)
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    positions = w.positions()
    c_prev = int(positions[0]) // 64
    layer.pool_blocks(kv, logits, 0, c_prev)
    sels, nsels, outs = [], [], []
    for t in range(n):
        c = int(positions[t]) // 64
        if c > c_prev:
            layer.pool_blocks(kv, logits, c_prev, c)
            c_prev = c
        if fused:
            layer.step_fused(qd[t], kv, pos[t])
        else:
            layer.step_resident(qd[t], kv, pos[t])
        sels.append(layer.sel.clone())
        nsels.append(layer.n_sel.clone())
        outs.append(layer.out.float().clone())
    torch.cuda.synchronize()
    return ([s.cpu().numpy() for s in sels], [s.cpu().numpy() for s in nsels],
            [o.cpu().numpy() for o in outs], layer)


def unit_selections(S_rows, N_rows, b, h) -> List[List[int]]:
    return [list(S[b, h, :N[b, h]]) for S, N in zip(S_rows, N_rows)]


def oracle_scores(w: NI.Workload, K, V, lam, q, b, h, positions=None, pool_slots=None, pool_reset_at=None):
    """Oracle per-step selection data for unit (b, h): s_q, E, own selections
    (and, with pool_slots, the pool replay of those selections)."""
    G = w.group
    qrows = q[:, b, h * G:(h + 1) * G]
    positions = w.positions() if positions is None else positions
    tr = O.decode_unit(K[b, h], V[b, h], lam[b, h], qrows, positions[: q.shape[0]], w.kq, w.ke,
                       bf16=(w.dtype == "bf16"), attend=False, pool_slots=pool_slots, pool_reset_at=pool_reset_at)
    E = O.block_eviction_scores(O.subblock_logit_means(lam[b, h]))
    return tr, E


def compare_unit(w: NI.Workload, K, V, lam, q, b, h, gpu_sel, gpu_out=None, gpu_pool=None, positions=None,
                 pool_reset_at=None):
    """Check one (b, h) unit of a GPU run against the oracle; returns stats.
    positions: the unit's own positions (default: the workload's);
    pool_reset_at: step at which the oracle's pool starts again empty."""
    G = w.group
    positions = w.positions() if positions is None else positions
    pool_slots = w.pool_slots if gpu_pool else None
    tr, E = oracle_scores(w, K, V, lam, q, b, h, positions, pool_slots, pool_reset_at)
    forced: Dict[int, List[int]] = {}
    ties = 0
    for t, S in enumerate(gpu_sel):
        c = int(positions[t]) // 64
        if list(S) != tr.sel[t]:
            assert selection_ok(S, tr.s_q[t], E, c, w.kq, w.ke), (
                f"unit ({b},{h}) step {t}: gpu {sorted(S)} oracle {tr.sel[t]}")
            forced[t] = list(S)
            ties += 1
        assert list(S) == sorted(S)
    if gpu_out is None and gpu_pool is None:
        return dict(ties=ties)
    if not forced and gpu_out is None and len(gpu_sel) == q.shape[0]:
        tr2 = tr          # the first run replayed the pool over the GPU's own sets
    else:
        qrows = q[:, b, h * G:(h + 1) * G]
        tr2 = O.decode_unit(K[b, h], V[b, h], lam[b, h], qrows, positions[: len(gpu_sel)], w.kq, w.ke,
                            bf16=(w.dtype == "bf16"), pool_slots=pool_slots,
                            attend=gpu_out is not None, forced_sel=forced, pool_reset_at=pool_reset_at)
    err = 0.0
    if gpu_out is not None:
        for t in range(len(gpu_sel)):
            ref = tr2.out[t]
            got = gpu_out[t][b, h * G:(h + 1) * G]
            e = float(np.max(np.abs(got - ref)))
            err = max(err, e)
            assert e <= ATOL[w.dtype], f"unit ({b},{h}) step {t}: max |err| {e}"
    return dict(ties=ties, max_err=err, trace=tr2)


def run_offload(w: NI.Workload, K, V, lam, q, steps: Optional[int] = None, side_stream: bool = True,
                record_tables: bool = True, offsets=None, reset_at: Optional[int] = None, fused_fetch: bool = False):
    """GPU decode in offload mode (KV in pinned host memory, HBM block pool).

    offsets: per batch entry, how many positions it lags the workload's
    (entry b decodes position p_t - offsets[b] at step t), so the entries'
    windows complete blocks on different steps: each step pools and inserts
    the blocks that just completed, per entry.  reset_at: before that step
    the pool tables are cleared (a cold restart: every resident block is
    forgotten, the compressed keys are kept).  fused_fetch: the gather folded
    into the attention (nosa_select_update_pool + nosa_sparse_decode_attn_fetch)."""
    n = w.n_steps if steps is None else steps
    kv_dev, logits, qd, _ = device_inputs(w, K, V, lam, q)
    offs = np.zeros(w.batch, np.int64) if offsets is None else np.asarray(offsets, np.int64)
    P = w.positions()[:n, None].astype(np.int64) - offs[None, :]          # [n, B]
    assert P.min() >= 0
    pos = torch.from_numpy(P.astype(np.int32)).cuda()
    host = kv_dev.cpu().pin_memory()
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq,
                          w.ke, pool_slots=w.pool_slots)
    C = P // 64                                                             # window block per step, entry
    c_prev = C[0].copy()
    lo = int(c_prev.min())
    layer.pool_blocks(kv_dev, logits, 0, lo)          # prefill: blocks complete for every entry
    for j in range(lo, int(c_prev.max())):            # and the ones complete for some entries only
        eb = torch.from_numpy(np.where(j < c_prev, j, -1).astype(np.int32)).cuda()
        layer.pool_entries(kv_dev, logits, eb)
    bidx = torch.arange(w.batch, device="cuda")
    blocks_of = lambda c: kv_dev[bidx, :, torch.from_numpy(c).cuda()]      # [B, Hkv, block]
    side = torch.cuda.Stream() if side_stream else None
    rec = {k: [] for k in ("sel", "n_sel", "out", "phys", "miss_list", "n_miss", "block_table", "slot_block")}
    for t in range(n):
        c = C[t]
        ins_blk = ins_src = None
        done = c > c_prev
        if done.any():
            ins_src = blocks_of(c_prev).contiguous()
            ins_blk = torch.from_numpy(np.where(done, c_prev, -1).astype(np.int32)).cuda()
            layer.pool_entries(ins_src, logits, ins_blk, layer.blk_elems, 0)
        if reset_at is not None and t == reset_at:
            for k in ("block_table", "slot_block", "slot_last_use"):
                getattr(layer, k).fill_(-1)
        window = blocks_of(c).contiguous()
        layer.step_offload(qd[t], host, window, pos[t], t, ins_blk, ins_src, side, fused_fetch)
        for k in ("sel", "n_sel", "phys", "miss_list", "n_miss"):
            rec[k].append(getattr(layer, k).clone())
        rec["out"].append(layer.out.float().clone())
        if record_tables:
            rec["block_table"].append(layer.block_table.clone())
            rec["slot_block"].append(layer.slot_block.clone())
        c_prev = c
    torch.cuda.synchronize()
    del kv_dev
    out = {k: [x.cpu().numpy() for x in v] for k, v in rec.items()}
    out["positions"] = P
    return out, layer, host


def check_offload_unit(w: NI.Workload, K, V, lam, q, rec, b, h, pool_reset_at=None, outputs: bool = True):
    """Oracle comparison of one unit of an offload run: selections, pool
    tables (miss list, insert entry, physical slots) and, unless outputs is
    False, the attention outputs."""
    positions = rec["positions"][:, b] if "positions" in rec else w.positions()[: len(rec["sel"])]
    sels = unit_selections(rec["sel"], rec["n_sel"], b, h)
    st = compare_unit(w, K, V, lam, q, b, h, sels, gpu_out=rec["out"] if outputs else None, gpu_pool=True,
                      positions=positions, pool_reset_at=pool_reset_at)
    tr = st["trace"]
    for t in range(len(sels)):
        nm = int(rec["n_miss"][t][b, h])
        ml = rec["miss_list"][t][b, h]
        got = [tuple(int(x) for x in ml[i]) for i in range(nm)]
        assert got == [tuple(m) for m in tr.misses[t]], (b, h, t, got, tr.misses[t])
        ins = tuple(int(x) for x in ml[w.kq + w.ke])
        exp_ins = (-1, -1) if tr.insert_slot[t] < 0 else (int(positions[t]) // 64 - 1, tr.insert_slot[t])
        assert ins == exp_ins, (b, h, t, ins, exp_ins)
        assert list(rec["phys"][t][b, h, : len(sels[t])]) == tr.phys[t]
    st["misses"] = sum(len(m) for m in tr.misses)
    return st
