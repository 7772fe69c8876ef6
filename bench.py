"""Benchmark of the NOSA decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-offload] [--no-cpu]

Headline: the layer32k workload (one attention layer, batch 8, 16 query /
2 KV heads, head_dim 128, bf16, 32K-token context, top-64 blocks of 64
tokens: kq = 16 query-aware + ke = 48 query-agnostic, plus the window),
synthetic seeded data.  A step is one decode token for the whole batch:
block selection and sparse attention, run as one launch of nosa_decode_step
(the separate nosa_select_blocks + nosa_sparse_decode_attn pair is timed too).
No block completes during these 64 positions, so nosa_pool_keys has nothing
to do (the offload leg exercises it).  Steps are captured in a HIP graph and
replayed.

Cold-cache protocol: a step touches about 42 MB (8.4 MB of compressed keys,
about 33 MB of selected blocks and the window), and consecutive steps share
most of it, so replicas of the layer's cache and compressed keys at distinct
addresses are rotated: step t uses replica t mod R, with R chosen so that the
bytes touched between two uses of one replica are at least twice the 256 MB
Infinity Cache, and so that the other replicas' compressed keys alone fill it
(the step reads the blocks with non-temporal loads, so the compressed keys are
what the caches keep): R = 33, 1.33 GB in between, 270 MB of it compressed
keys, 8.9 GB of caches in rotation, about the KV cache of a 32-layer model of
this shape.  The same steps on one replica are reported too, labelled warm;
`value` and the roofline are the cold ones.

Prints ONE JSON line.  Extra objects: roofline of the dominant kernel
(step_kernel, the one launch of a step), per-kernel times, the two variant
readings beside the path's own (fill-the-remainder selection: Jaccard, set
sizes, re-admissions, output deltas; eviction-logit bias: output deltas) on
layer32k and on the offload workload, the offload leg (KV in pinned host
memory, HBM pool of 80 blocks per KV head, the offload workload, the kq/k
sweep and the transfer operator's blocks-per-call sweep), the 28-layer
stack, the prefill leg, the QKV split and the oracle's CPU baseline on a
bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
INFINITY_CACHE_BYTES = 256 << 20
COLD_FACTOR = 2.0           # bytes touched between two uses of a replica >= 2x the Infinity Cache
KEPT_FACTOR = 1.0           # ... and the selection's bytes (compressed keys, scores) alone >= 1x
# Byte counters of step_kernel on this workload (rocprofv3 --pmc, KiB per dispatch),
# valid for the kernel sources whose digest is recorded here.  FETCH_SIZE reads half
# of a plain 256 MiB copy's bytes (factor 2.0); WRITE_SIZE reads all of them (1.0).
STEP_PMC = {"src_sha256": "af700ed005f01f21a29223ad4f1e4c96b7123b82902ea2884a0b3f69cf63785e", "fetch_kib": 21804.4, "write_kib": 2225.0}
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0
STEP_SOURCES = ("fused.hip", "attn_dev.h", "select_dev.h", "nosa_common.h")


def kernel_source_digest():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(os.path.join(here, "kv_cache_offload_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-offload", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 28-layer offload stack (about 2 min of input generation)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch each step instead of graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of 256 MiB, three times: the reference that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(w, n_sel_rows, positions):
    """Algorithmic HBM bytes of the steps whose per-unit n_S are given.

    Per (b, KV head): q 2GD + compressed-key scan 4c*D*2 + block scores 4c +
    selected K,V n_S*64*2D*2 + window (p-64c+1)*2D*2 + output 2GD (bytes,
    bf16); the selected ids (4 bytes each) are counted with the attention.
    """
    G, D = w.group, w.head_dim
    sel_b, attn_b = [], []
    for n_s, p in zip(n_sel_rows, positions):
        c = int(p) // 64
        win = int(p) - 64 * c + 1
        units = n_s.size
        qb = G * D * 2
        sel_b.append(units * (qb + 4 * c * D * 2 + 4 * c) + int(n_s.sum()) * 4)
        attn_b.append(units * (qb + win * 2 * D * 2 + qb) + int(n_s.sum()) * (64 * 2 * D * 2 + 4))
    return np.array(sel_b, np.float64), np.array(attn_b, np.float64)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on a single GPU (no sharding is implemented); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import nosa_inputs as NI
    from kv_cache_offload_amd import binding as nb
    from kv_cache_offload_amd import runner as R

    # ------------------------------------------------------------ inputs
    w = NI.WORKLOADS["layer32k"]
    t0 = time.perf_counter()
    K, V, lam, q = NI.layer_inputs(w)
    log(f"inputs {w.name}: {time.perf_counter() - t0:.1f}s")
    # the oracle's CPU baseline runs first: its worker processes are forked
    # before this process touches the GPU
    cpu_baseline = None if args.no_cpu else _cpu_baseline(NI, w, K, V, lam, q)

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    nb.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kv0, logits, qd, pos = _device_inputs(w, K, V, lam, q, R)
    c0 = int(w.positions()[0]) // 64
    n_pos = w.n_steps
    positions = w.positions()
    assert all(int(p) // 64 == c0 for p in positions), "no block completes in the headline workload"

    def new_layer(kv):
        L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
        L.pool_blocks(kv, logits, 0, c0)
        return L

    # untimed pass on one replica: warm-up and the per-step n_S for the byte count
    kvs, layers = [kv0], [new_layer(kv0)]
    n_sel_rows = []
    for t in range(max(args.steps, args.warmup)):
        layers[0].step_fused(qd[t % n_pos], kv0, pos[t % n_pos])
        if t < args.steps:
            n_sel_rows.append(layers[0].n_sel.cpu().numpy().copy())
    torch.cuda.synchronize()
    pos_steps = [positions[t % n_pos] for t in range(args.steps)]
    sel_bytes, attn_bytes = step_bytes(w, n_sel_rows, pos_steps)
    step_b = float((sel_bytes + attn_bytes).mean())
    # cold: enough replicas that the bytes the other replicas' steps touch
    # between two uses of one replica are >= COLD_FACTOR x the Infinity Cache,
    # and their compressed keys (read with plain loads, unlike the blocks)
    # alone >= KEPT_FACTOR x
    sel_b = float(sel_bytes.mean())
    n_rep = max(16, 1 + math.ceil(COLD_FACTOR * INFINITY_CACHE_BYTES / step_b),
                1 + math.ceil(KEPT_FACTOR * INFINITY_CACHE_BYTES / sel_b))
    for r in range(1, n_rep):
        kvs.append(kv0.clone())
        layers.append(new_layer(kvs[r]))
    between_mb = (n_rep - 1) * step_b / 1e6
    kept_mb = (n_rep - 1) * sel_b / 1e6
    log(f"cold protocol: {n_rep} replicas, {between_mb:.0f} MB touched between two uses of one replica, "
        f"{kept_mb:.0f} MB of it compressed keys and scores")

    def step(t, stream=None, n_r=n_rep):
        r = t % n_r
        i = t % n_pos
        layers[r].step_fused(qd[i], kvs[r], pos[i], stream)

    def step_separate(t, stream=None):
        r = t % n_rep
        i = t % n_pos
        layers[r].step_resident(qd[i], kvs[r], pos[i], stream)

    for t in range(n_rep):
        step(t)                         # every replica's step workspace initialised
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for t in range(2):           # warm the capture stream
                fn(t)
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for t in range(n):
                    fn(t)
        return g

    def time_graph(g, reps=20):
        """Median ms of one replay over `reps` replays (events on the replay stream)."""
        times = []
        with torch.cuda.stream(stream):
            g.replay()
            stream.synchronize()
            for _ in range(reps):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                b.synchronize()
                times.append(a.elapsed_time(b))
        return float(np.median(times)), float(np.percentile(times, 10)), float(np.percentile(times, 90))

    K_steps = args.steps
    if args.eager:
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            for t in range(args.warmup):
                step(t, stream)
            a.record(stream)
            for t in range(K_steps):
                step(t, stream)
            b.record(stream)
        b.synchronize()
        total_ms = a.elapsed_time(b)
        p10 = p90 = total_ms
        warm_ms = float("nan")
    else:
        g_step = capture(lambda t: step(t, stream), K_steps)
        total_ms, p10, p90 = time_graph(g_step)
        # warm: the same steps, every one on replica 0
        g_warm = capture(lambda t: step(t, stream, 1), K_steps)
        warm_ms = time_graph(g_warm)[0]
    torch.cuda.synchronize()
    ms_per_step = total_ms / K_steps
    warm_ms_per_step = warm_ms / K_steps

    # per-kernel averages: graphs holding only one kernel, same arguments (cold rotation)
    def sel_only(t):
        r = t % n_rep
        layers[r].select(qd[t % n_pos], pos[t % n_pos], stream)

    def attn_only(t):
        r = t % n_rep
        layers[r].attend_resident(qd[t % n_pos], kvs[r], pos[t % n_pos], stream)

    g_sel = capture(sel_only, K_steps)
    sel_ms = time_graph(g_sel)[0] / K_steps
    g_attn = capture(attn_only, K_steps)
    attn_ms = time_graph(g_attn)[0] / K_steps
    g_sep = capture(lambda t: step_separate(t, stream), K_steps)
    sep_ms = time_graph(g_sep)[0] / K_steps
    # the two variant calls, same rotation
    g_self = capture(lambda t: layers[t % n_rep].select(qd[t % n_pos], pos[t % n_pos], stream, fill=True), K_steps)
    sel_fill_ms = time_graph(g_self)[0] / K_steps
    g_attb = capture(lambda t: layers[t % n_rep].attend_resident_bias(qd[t % n_pos], kvs[t % n_rep], pos[t % n_pos],
                                                                        logits, stream), K_steps)
    attn_bias_ms = time_graph(g_attb)[0] / K_steps
    # bounded hand-off waits of the one-launch step that hit their bound in any
    # of the timed launches (each spoils that launch's outputs)
    timeouts = sum(L.step_timeouts() for L in layers)

    traffic = None
    if STEP_PMC["src_sha256"] == kernel_source_digest():
        traffic = int(STEP_PMC["fetch_kib"] * 1024 * FETCH_FACTOR + STEP_PMC["write_kib"] * 1024 * WRITE_FACTOR)
    tok_per_s = w.batch / (ms_per_step * 1e-3)
    hbm_gbps = step_b / (ms_per_step * 1e-3) / 1e9
    warm_gbps = step_b / (warm_ms_per_step * 1e-3) / 1e9
    attn_gbps = float(attn_bytes.mean()) / (attn_ms * 1e-3) / 1e9
    sel_gbps = float(sel_bytes.mean()) / (sel_ms * 1e-3) / 1e9
    log(f"step (one launch) {ms_per_step * 1e3:.2f} us cold, {warm_ms_per_step * 1e3:.2f} us warm; separate calls "
        f"{sep_ms * 1e3:.2f} us (select {sel_ms * 1e3:.2f} us + attention {attn_ms * 1e3:.2f} us); "
        f"hand-off timeouts {timeouts}")

    result = {
        "metric": "decode tokens/s at 32K ctx (bf16, top-64x64-tok blocks) + achieved HBM GB/s",
        "value": round(tok_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "ms_per_step_p10_p90": [round(p10 / K_steps, 6), round(p90 / K_steps, 6)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; keys N(0,1)+per-block N(0,0.5^2) offset, values N(0,1), AR(1) rho=0.9 queries)",
        "config": {"workload": "layer32k", "batch": w.batch, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "context": w.prompt_len,
                   "kq": w.kq, "ke": w.ke, "block": 64, "layers": 1,
                   "cache_replicas": n_rep, "graph": not args.eager},
        "timing": {"cold": f"{n_rep} replicas rotated: {between_mb:.0f} MB touched between two uses of one replica "
                           f"({between_mb * 1e6 / INFINITY_CACHE_BYTES:.1f}x the 256 MB Infinity Cache), "
                           f"{kept_mb:.0f} MB of it compressed keys and scores "
                           f"({kept_mb * 1e6 / INFINITY_CACHE_BYTES:.2f}x)",
                   "warm": "every step on one replica"},
        "hbm_gbps": round(hbm_gbps, 1),
        "hbm_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "step_bytes": int(step_b),
        "warm": {"ms_per_step": round(warm_ms_per_step, 6),
                 "tokens_per_s": round(w.batch / (warm_ms_per_step * 1e-3), 1),
                 "hbm_gbps": round(warm_gbps, 1), "hbm_frac": round(warm_gbps / HBM_PEAK_GBPS, 4)},
        "step_timeouts": int(timeouts),
        "kernels": {"step_kernel_us": round(ms_per_step * 1e3, 3),
                    "separate_calls_step_us": round(sep_ms * 1e3, 3),
                    "select_us": round(sel_ms * 1e3, 3), "select_gbps": round(sel_gbps, 1),
                    "attn_us": round(attn_ms * 1e3, 3), "attn_gbps": round(attn_gbps, 1)},
        "roofline": {"kernel": "nosa step_kernel (selection + sparse attention, one launch per step)",
                     "bound": "hbm", "achieved": round(hbm_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": int(step_b)},
    }
    result["kernels"].update({"select_fill_us": round(sel_fill_ms * 1e3, 3),
                              "attn_bias_us": round(attn_bias_ms * 1e3, 3)})
    t0 = time.perf_counter()
    result["variants"] = _variants(torch, nb, layers[0], kvs[0], logits, qd, pos, range(n_pos))
    log(f"variants layer32k ({time.perf_counter() - t0:.1f}s): {json.dumps(result['variants'])}")
    del layers, kvs

    if not args.no_offload:
        result["offload"] = _offload_leg(torch, NI, R, nb)
        torch._C._host_emptyCache()          # hand the offload leg's pinned cache back
    if not args.no_prefill:
        result["prefill"] = _prefill_leg(torch, NI, R, nb)
        result["split_qkv"] = _split_leg(torch, nb)
    if not args.no_stack:
        try:
            result["stack"] = _stack_leg(torch, NI, R)
        except RuntimeError as e:            # e.g. not enough pinned host memory for 56 GiB of caches
            log(f"stack leg failed: {e}")
            result["stack"] = {"workload": "stack128k", "error": str(e).splitlines()[0][:200]}
    if cpu_baseline is not None:
        result["cpu_baseline"] = cpu_baseline
    print(json.dumps(result), flush=True)
    if timeouts:
        log(f"{timeouts} hand-off waits of the one-launch step hit their bound: those launches' outputs are wrong")
        sys.exit(3)


def _device_inputs(w, K, V, lam, q, R):
    import torch
    NB = w.n_blocks
    kv = R.to_device_blocks(K, V, NB, w.dtype)
    logits = R.pad_logits(torch.from_numpy(lam).cuda(), NB)
    qd = torch.from_numpy(q).cuda().to(R.torch_dtype(w.dtype))
    pos = torch.from_numpy(np.repeat(w.positions()[:, None], w.batch, axis=1).astype(np.int32)).cuda()
    return kv, logits, qd, pos


KQ_SWEEP = (8, 16, 32, 64)        # kq at k = kq + ke = 64: kq/k = 0.125, 0.25, 0.5, 1.0


def _offload_run(torch, R, w, kq, ke, kv_dev, host, windows, logits, qd, pos, fill=False, fused_fetch=False):
    """One offload decode run from a cold pool; per-step events, no host sync
    inside the loop (fill: the selection under the other reading of Eq. 7;
    fused_fetch: the gather folded into the attention, one stream).  Returns
    step and gather times (ms; with fused_fetch, the attention's, which holds
    the gather), misses, set sizes and selections per step."""
    positions = w.positions()
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, kq, ke,
                          pool_slots=w.pool_slots)
    c_prev = int(positions[0]) // 64
    layer.pool_blocks(kv_dev, logits, 0, c_prev)       # prefill: compressed keys of the prompt
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev, rec = [], []
    for t in range(w.n_steps):
        c = int(positions[t]) // 64
        ins_blk = ins_src = None
        e0, e1, f0, f1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        e0.record(main)
        if c > c_prev:
            layer.pool_window(windows[c_prev], logits, c_prev, main)
            ins_blk = torch.full((w.batch,), c_prev, dtype=torch.int32, device="cuda")
            ins_src = windows[c_prev]
        # selection and pool update (one launch; two for the fill variant),
        # then the gather on the side stream while the attention over the
        # blocks already resident runs (the runner's offload step)
        if fill:
            layer.select(qd[t], pos[t], main, fill=True)
            layer.update_pool(t, ins_blk, main)
        else:
            layer.select_update(qd[t], pos[t], t, ins_blk, main)
        if fused_fetch:
            f0.record(main)
            layer.attend_fetch(qd[t], host, windows[c], pos[t], ins_src, main)
            f1.record(main)
        else:
            side.wait_stream(main)
            f0.record(side)
            layer.gather(host, ins_src, side)
            f1.record(side)
            layer.attend_pool_part(qd[t], windows[c], pos[t], 0, main)
            main.wait_stream(side)
            layer.attend_pool_part(qd[t], windows[c], pos[t], 1, main)
        e1.record(main)
        ev.append((e0, e1, f0, f1))
        rec.append((layer.n_miss.clone(), layer.n_sel.clone(), layer.sel.clone()))
        c_prev = c
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b, _, _ in ev])
    fetch_ms = np.array([a.elapsed_time(b) for _, _, a, b in ev])
    misses = np.array([int(m.sum().item()) for m, _, _ in rec])
    nsel = [n.cpu().numpy() for _, n, _ in rec]
    sels = [x.cpu().numpy() for _, _, x in rec]
    return step_ms, fetch_ms, misses, nsel, sels


def _offload_leg(torch, NI, R, nb):
    """The offload workload: KV in pinned host memory, HBM pool of 80 blocks
    per KV head, kq = 16 + ke = 48; then the kq/k sweep at k = 64 on the same
    inputs (each point from a cold pool)."""
    w = NI.WORKLOADS["offload"]
    t0 = time.perf_counter()
    K, V, lam, q = NI.layer_inputs(w, workers=NI.host_workers())
    log(f"inputs {w.name}: {time.perf_counter() - t0:.1f}s")
    kv_dev, logits, qd, pos = _device_inputs(w, K, V, lam, q, R)
    del K, V
    host = torch.empty(kv_dev.shape, dtype=kv_dev.dtype, pin_memory=True)
    host.copy_(kv_dev)
    positions = w.positions()
    windows = {c: kv_dev[:, :, c].clone() for c in sorted({int(p) // 64 for p in positions})}
    torch.cuda.synchronize()
    link_ref = _memcpy_h2d_gbps(torch, host)
    blocks = [int(p) // 64 for p in positions]
    blk_bytes = 2 * 64 * w.head_dim * 2
    units = w.batch * w.n_kv_heads
    warm = slice(1, None)                      # step 0 fills the cold pool

    def summary(kq, ke, step_ms, fetch_ms, misses, nsel, sels):
        ms = float(np.median(step_ms[warm]))
        miss_bytes = misses.astype(np.float64) * blk_bytes
        link = float(miss_bytes[warm].sum() / (fetch_ms[warm].sum() * 1e-3) / 1e9)
        # algorithmic HBM bytes of a step (the resident path's, with the misses
        # also written into the pool), from the logged set sizes and misses
        sb, ab = step_bytes(w, nsel, list(positions[: len(nsel)]))
        hbm = float(np.mean((sb + ab + miss_bytes)[warm])) / (ms * 1e-3) / 1e9
        return {
            "kq": kq, "ke": ke, "kq_over_k": round(kq / (kq + ke), 4),
            "tokens_per_s": round(w.batch / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "ms_per_step_p10_p90": [round(float(np.percentile(step_ms[warm], 10)), 4),
                                    round(float(np.percentile(step_ms[warm], 90)), 4)],
            "cold_step_ms": round(float(step_ms[0]), 4),
            "misses_per_unit_step": round(float(misses[warm].mean()) / units, 3),
            "miss_fraction": round(float(misses[warm].sum() / sum(n.sum() for n in nsel[1:])), 4),
            "locality_gamma": round(_locality(sels, nsel, blocks), 4),
            "host_link_gbps": round(link, 2), "host_link_frac_of_memcpy": round(link / link_ref, 4),
            "hbm_gbps": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBPS, 4),
            "cold_step_host_link_gbps": round(float(miss_bytes[0] / (fetch_ms[0] * 1e-3) / 1e9), 2),
            "gather_share_of_step": round(float(fetch_ms[warm].sum() / step_ms[warm].sum()), 4),
        }

    # the GPU's mapping of the pinned cache touched once before anything is timed
    L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke,
                      pool_slots=w.pool_slots)
    t0 = time.perf_counter()
    warm_rates = _warm_host_mapping(torch, nb, L, host, w.n_blocks)
    sweep = _transfer_sweep(torch, nb, L, host, blocks[0])
    log(f"host cache warm-up passes (GB/s): {', '.join(f'{r:.1f}' for r in warm_rates)}")
    log(f"transfer sweep ({time.perf_counter() - t0:.1f}s, memcpy {link_ref:.1f} GB/s): " +
        ", ".join(f"{n}: {g:.1f}" for n, _, g in sweep))
    del L

    points = []
    for kq in KQ_SWEEP:
        ke = 64 - kq
        pt = summary(kq, ke, *_offload_run(torch, R, w, kq, ke, kv_dev, host, windows, logits, qd, pos,
                                           fused_fetch=True))
        log(f"offload kq={kq:2d} ke={ke:2d}: step {pt['ms_per_step']:.3f} ms, misses/unit/step "
            f"{pt['misses_per_unit_step']:.2f}, gamma {pt['locality_gamma']:.3f}, link {pt['host_link_gbps']:.1f} GB/s")
        points.append(pt)
    main_pt = next(p for p in points if p["kq"] == w.kq and p["ke"] == w.ke)
    out = {"workload": "offload", "batch": w.batch, "context": w.prompt_len, "pool_slots": w.pool_slots,
           "steps": w.n_steps, "graph": False, "memcpy_h2d_gbps": round(link_ref, 2),
           "step": "selection + pool update (one launch), then the attention with the gather folded in; "
                   "host_link_gbps: miss bytes / that attention's time"}
    out.update(main_pt)
    out["kq_sweep"] = [{k: v for k, v in p.items() if k not in ("ms_per_step_p10_p90",)} for p in points]
    out["host_warmup_pass_gbps"] = [round(r, 2) for r in warm_rates]
    out["transfer_sweep"] = {
        "call": "nosa_gather_blocks alone, n blocks of 32 KiB per call spread over the 128 units, each block "
                "read once per call size; median of 20 calls",
        "points": [{"blocks": n, "us": round(us, 2), "gbps": round(g, 2), "frac_of_memcpy": round(g / link_ref, 4)}
                   for n, us, g in sweep]}
    # the same step with the gather on a side stream beside the attention over
    # the resident blocks, then the attention over the fetched ones
    ss = summary(w.kq, w.ke, *_offload_run(torch, R, w, w.kq, w.ke, kv_dev, host, windows, logits, qd, pos))
    out["gather_on_side_stream"] = {k: ss[k] for k in ("tokens_per_s", "ms_per_step", "ms_per_step_p10_p90",
                                                       "cold_step_ms", "misses_per_unit_step", "host_link_gbps",
                                                       "gather_share_of_step")}
    log(f"offload, gather on a side stream, kq={w.kq}: step {ss['ms_per_step']:.3f} ms, "
        f"link {ss['host_link_gbps']:.1f} GB/s")
    # the other reading of Eq. 7 through the same offload step, and both variants step by step
    fp = summary(w.kq, w.ke, *_offload_run(torch, R, w, w.kq, w.ke, kv_dev, host, windows, logits, qd, pos,
                                           fill=True, fused_fetch=True))
    L = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype, w.kq, w.ke)
    L.pool_blocks(kv_dev, logits, 0, blocks[-1])
    var = _variants(torch, nb, L, kv_dev, logits, qd, pos, range(w.n_steps))
    var["fill_offload"] = {k: fp[k] for k in ("ms_per_step", "misses_per_unit_step", "miss_fraction",
                                              "locality_gamma", "host_link_gbps")}
    out["variants"] = var
    log(f"variants offload: {json.dumps(var)}")
    del L
    del windows, kv_dev
    return out


def _memcpy_h2d_gbps(torch, host):
    """Rate of one 1 GiB pinned host -> HBM copy (the host-link reference)."""
    src = host.reshape(-1)[: (1 << 29)]
    dst = torch.empty_like(src, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    dst.copy_(src, non_blocking=True)
    b.record()
    b.synchronize()
    return src.numel() * src.element_size() / (a.elapsed_time(b) * 1e-3) / 1e9


def _locality(sels, nsels, blocks):
    """Mean over steps t >= 1 and units of the block-level overlap
    |S(t) & (S(t-1) | {window block of t-1})| / |S(t)| (steps with an empty
    S(t) are skipped)."""
    vals = []
    for t in range(1, len(sels)):
        prev, cur = sels[t - 1], sels[t]
        for idx in np.ndindex(cur.shape[:-1]):
            n = int(nsels[t][idx])
            if n == 0:
                continue
            a = set(cur[idx][:n].tolist())
            b = set(prev[idx][: int(nsels[t - 1][idx])].tolist()) | {blocks[t - 1]}
            vals.append(len(a & b) / n)
    return float(np.mean(vals)) if vals else float("nan")


def _readmissions(parts):
    """Blocks that come back into a unit's query-agnostic part after having
    left it, summed over the steps; `parts` is that part's block set per step.
    The eviction rule (a block pushed out of that part never returns) makes
    this 0 under the path's reading of Eq. 7."""
    dropped, count = set(), 0
    for t, cur in enumerate(parts):
        count += len(cur & dropped)
        if t:
            dropped |= parts[t - 1] - cur
        dropped -= cur
    return count


def _variants(torch, nb, L, kv, logits, qd, pos, steps):
    """The two alternative readings beside the path's own, step by step on one
    layer whose compressed keys cover every candidate of the given steps
    (nothing timed here):

      * Eq. 7 as "fill the remainder from the candidates left"
        (nosa_select_blocks_fill) against the union Gamma_q | Gamma_e: Jaccard
        of the two sets, their sizes, the re-admissions of each reading's
        query-agnostic part (Gamma_e for the union, S \\ Gamma_q for the fill;
        Gamma_q and Gamma_e come from the same selection kernel run with one
        budget at 0), and the attention output over the fill set against the
        one over the union set;
      * ED-DMA's logits as an attention bias (nosa_sparse_decode_attn_bias)
        against the plain attention, both over the union set.

    Output deltas are max |delta| and ||delta||_2 / ||out||_2 per step."""
    kq, ke = L.kq, L.ke
    z = dict(device="cuda")

    def one_budget(a, b):
        ws = torch.zeros(max(nb.workspace_size(L.dims, nb.OP_SELECT, 1, a, b), 1), dtype=torch.uint8, **z)
        s = torch.full((L.B, L.Hkv, max(a + b, 1)), -1, dtype=torch.int32, **z)
        n = torch.zeros((L.B, L.Hkv), dtype=torch.int32, **z)
        return lambda t: (nb.select_blocks(L.dims, qd[t], 1, pos[t], L.k_comp, L.e_blk, a, b, s, n, ws), s, n)

    sel_q, sel_e = one_budget(kq, 0), one_budget(0, ke)

    def sets(s, n):
        s, n = s.cpu().numpy(), n.cpu().numpy()
        return {u: set(s[u][: n[u]].tolist()) for u in np.ndindex(n.shape)}

    def delta(a, b):
        d = (a - b).abs()
        return float(d.max()), float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b).clamp_min(1e-30))

    jac, n_u, n_f, bias_d, fill_d, broken = [], [], [], [], [], 0
    part_u, part_f = {}, {}
    for t in steps:
        L.select(qd[t], pos[t])
        S_u = sets(L.sel, L.n_sel)
        L.attend_resident(qd[t], kv, pos[t])
        out_u = L.out.float().clone()
        L.attend_resident_bias(qd[t], kv, pos[t], logits)
        bias_d.append(delta(L.out.float(), out_u))
        L.select(qd[t], pos[t], fill=True)
        S_f = sets(L.sel, L.n_sel)
        L.attend_resident(qd[t], kv, pos[t])
        fill_d.append(delta(L.out.float(), out_u))
        G_q = sets(*sel_q(t)[1:])
        G_e = sets(*sel_e(t)[1:])
        for u in S_u:
            if S_u[u] != G_q[u] | G_e[u]:
                broken += 1
            jac.append(len(S_u[u] & S_f[u]) / max(len(S_u[u] | S_f[u]), 1))
            n_u.append(len(S_u[u]))
            n_f.append(len(S_f[u]))
            part_u.setdefault(u, []).append(G_e[u])
            part_f.setdefault(u, []).append(S_f[u] - G_q[u])
    torch.cuda.synchronize()
    if broken:
        raise RuntimeError(f"{broken} union sets differ from Gamma_q | Gamma_e of the one-budget selections")
    units = len(part_u)
    re_u = sum(_readmissions(p) for p in part_u.values())
    re_f = sum(_readmissions(p) for p in part_f.values())
    bd, fd = np.array(bias_d), np.array(fill_d)
    return {
        "steps": len(steps), "units": units,
        "fill_vs_union": {
            "jaccard_mean": round(float(np.mean(jac)), 4), "jaccard_min": round(float(np.min(jac)), 4),
            "set_size_union_mean": round(float(np.mean(n_u)), 3), "set_size_fill_mean": round(float(np.mean(n_f)), 3),
            "readmissions_union": int(re_u), "readmissions_fill": int(re_f),
            "readmissions_fill_per_unit_step": round(re_f / (units * len(steps)), 4),
            "output_max_abs_delta": round(float(fd[:, 0].max()), 5),
            "output_rel_l2_delta_mean": round(float(fd[:, 1].mean()), 5)},
        "bias_vs_plain": {
            "output_max_abs_delta": round(float(bd[:, 0].max()), 5),
            "output_rel_l2_delta_mean": round(float(bd[:, 1].mean()), 5)},
    }


def _transfer_sweep(torch, nb, L, host, n_blocks, reps=20):
    """The gather alone (nosa_gather_blocks) at 1 ... 1024 blocks per call:
    per call, `n` misses spread over the units (unit u takes n // units, plus
    one if u < n % units), each from a block no earlier call of the same size
    read, into pool slots 0, 1, ...  Median over `reps` calls (events around
    each).  Returns [(n, us, GB/s)]."""
    units = L.B * L.Hkv
    k1 = L.k + 1
    blk_bytes = L.blk_elems * host.element_size()
    ml = torch.full((units, k1, 2), -1, dtype=torch.int32)
    out = []
    for n in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
        per = np.array([n // units + (u < n % units) for u in range(units)], np.int32)
        assert per.max() <= L.k and per.max() <= L.pool_slots
        calls = []
        for r in range(reps + 2):                 # two untimed calls first
            m = ml.clone()
            for u in np.nonzero(per)[0]:
                e = np.arange(per[u])
                m[u, e, 0] = torch.from_numpy(((r * per[u] + e) % n_blocks).astype(np.int32))
                m[u, e, 1] = torch.from_numpy(e.astype(np.int32))
            calls.append(m.cuda())
        n_miss = torch.from_numpy(per).cuda()
        times = []
        for r, m in enumerate(calls):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            nb.gather_blocks(L.dims, host, L.pool, L.pool_slots, L.k, None, m, n_miss)
            b.record()
            b.synchronize()
            if r >= 2:
                times.append(a.elapsed_time(b))
        us = float(np.median(times)) * 1e3
        out.append((n, us, n * blk_bytes / (us * 1e-6) / 1e9))
    return out


def _warm_host_mapping(torch, nb, L, host, n_blocks, max_passes=8):
    """Untimed-in-the-results gathers of every block of the host cache (64
    blocks of each unit per call), pass after pass until two passes in a row
    agree within 5%: the first GPU reads of a pinned page run at about half
    the link rate, which would otherwise show up in whichever cold step
    comes first.  Returns each pass's GB/s."""
    units = L.B * L.Hkv
    k = min(L.k, L.pool_slots)
    calls = []
    for b0 in range(0, n_blocks, k):
        n = min(k, n_blocks - b0)
        m = torch.full((units, L.k + 1, 2), -1, dtype=torch.int32)
        m[:, :n, 0] = torch.arange(b0, b0 + n, dtype=torch.int32)
        m[:, :n, 1] = torch.arange(n, dtype=torch.int32)
        calls.append((m.cuda(), torch.full((units,), n, dtype=torch.int32, device="cuda")))
    nbytes = units * n_blocks * L.blk_elems * host.element_size()
    rates = []
    for _ in range(max_passes):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for m, n_miss in calls:
            nb.gather_blocks(L.dims, host, L.pool, L.pool_slots, L.k, None, m, n_miss)
        b.record()
        b.synchronize()
        rates.append(nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        if len(rates) >= 2 and abs(rates[-1] - rates[-2]) <= 0.05 * rates[-1]:
            break
    return rates


def _stack_leg(torch, NI, R):
    """The stack128k workload: 28 layers, batch 16, 131072-token context, each
    layer's KV cache in pinned host memory (2 GiB per layer) with an HBM pool
    of 80 blocks per KV head.  A decode step runs the layers in order, each
    select -> fetch (side stream) -> attention.  The pools start empty, so
    step 0 (cold, 64 misses per KV head per layer) is reported apart."""
    w = NI.WORKLOADS["stack128k"]
    workers = NI.host_workers()
    positions = w.positions()
    blocks = [int(p) // 64 for p in positions]
    stack = R.OffloadStack(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_blocks, w.dtype,
                           w.kq, w.ke, w.pool_slots)
    qs = []
    t0 = time.perf_counter()
    for l in range(w.n_layers):
        K, V, lam, q = NI.layer_inputs(w, l, workers=workers)
        stack.load_layer(l, K, V, lam, blocks[0], sorted(set(blocks)))
        qs.append(torch.from_numpy(q).cuda().to(R.torch_dtype(w.dtype)))
        del K, V, lam
        if l % 4 == 3 or l == w.n_layers - 1:
            log(f"stack: {l + 1} layers loaded, {time.perf_counter() - t0:.0f}s")
    setup_s = time.perf_counter() - t0
    pos = torch.from_numpy(np.repeat(positions[:, None], w.batch, axis=1).astype(np.int32)).cuda()
    torch.cuda.synchronize()
    link_ref = _memcpy_h2d_gbps(torch, stack.host[0])

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def run(fused_update, fused_fetch=False, record=False):
        """The decode steps from empty pools (tables cleared, window back at
        the prompt's end; the compressed keys of blocks completed on the way
        are pooled again, to the same values).  record: also copy every
        layer's sets and misses and time its gather (copies that would
        otherwise sit inside the timed steps)."""
        for L in stack.layers:
            for k in ("block_table", "slot_block", "slot_last_use"):
                getattr(L, k).fill_(-1)
        stack.block = blocks[0]
        torch.cuda.synchronize()
        fetch_ev = [[] for _ in range(w.n_layers)]
        step_ev = []
        rec = ([], [], [])

        def on_layer(l, L):
            rec[0].append(L.sel.clone())
            rec[1].append(L.n_sel.clone())
            rec[2].append(L.n_miss.clone())

        for t in range(w.n_steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(main)
            stack.step(t, [qd[t] for qd in qs], pos[t], blocks[t], side, on_layer if record else None,
                       fetch_ev if record else None, fused_update, fused_fetch)
            e1.record(main)
            step_ev.append((e0, e1))
        torch.cuda.synchronize()
        return fetch_ev, step_ev, rec

    # the selection and the pool update as two launches, then as one; then
    # also the gather folded into the attention (reported)
    med = lambda ev: float(np.median(np.array([a.elapsed_time(b) for a, b in ev])[1:]))
    ms_two = med(run(False)[1])
    ms_side = med(run(True)[1])
    _, step_ev, _ = run(True, True)
    # the same steps once more, recording each layer's sets, misses and
    # attention time (not timed as steps)
    fetch_ev, _, (rec_sel, rec_n, rec_miss) = run(True, True, record=True)
    nL = w.n_layers
    step_ms = np.array([a.elapsed_time(b) for a, b in step_ev])
    fetch_ms = np.array([[a.elapsed_time(b) for a, b in fetch_ev[l]] for l in range(nL)]).T   # [t, l]
    n_sel = np.stack([x.cpu().numpy() for x in rec_n]).reshape(w.n_steps, nL, w.batch, w.n_kv_heads)
    n_miss = np.stack([x.cpu().numpy() for x in rec_miss]).reshape(w.n_steps, nL, w.batch, w.n_kv_heads)
    sels = np.stack([x.cpu().numpy() for x in rec_sel]).reshape(w.n_steps, nL, w.batch, w.n_kv_heads, -1)
    gamma = _locality([sels[t] for t in range(w.n_steps)], [n_sel[t] for t in range(w.n_steps)], blocks)

    blk_bytes = 2 * 64 * w.head_dim * 2
    warm = slice(1, None)
    ms = float(np.median(step_ms[warm]))
    # algorithmic HBM bytes of the warm steps, per layer-step, from the logged set sizes and misses
    hbm = []
    for t in range(1, w.n_steps):
        sb, ab = step_bytes(w, list(n_sel[t]), [positions[t]] * nL)
        hbm.append(sb.sum() + ab.sum() + n_miss[t].sum() * blk_bytes)     # + pool writes
    hbm_gbps = float(np.mean(hbm)) / (ms * 1e-3) / 1e9
    miss_bytes = n_miss.sum(axis=(2, 3)).astype(np.float64) * blk_bytes          # [t, l]
    link = float(miss_bytes[warm].sum() / (fetch_ms[warm].sum() * 1e-3) / 1e9)
    cold_link = float(miss_bytes[0].sum() / (fetch_ms[0].sum() * 1e-3) / 1e9)
    fetch_share = float(fetch_ms[warm].sum() / step_ms[warm].sum())
    log(f"stack: step {ms:.3f} ms ({ms / nL * 1e3:.1f} us per layer; gather on a side stream: {ms_side:.3f} ms, "
        f"and with the selection and the pool update as two launches {ms_two:.3f} ms), cold step {step_ms[0]:.2f} ms, "
        f"misses/unit/layer-step {n_miss[warm].mean():.2f}, gamma {gamma:.3f}, link {link:.1f} GB/s "
        f"(cold {cold_link:.1f}; memcpy {link_ref:.1f}), HBM {hbm_gbps:.0f} GB/s")
    return {
        "workload": "stack128k", "layers": nL, "batch": w.batch, "context": w.prompt_len,
        "pool_slots": w.pool_slots, "steps": w.n_steps, "graph": False,
        "tokens_per_s": round(w.batch / (ms * 1e-3), 1),
        "layer_tokens_per_s": round(w.batch * nL / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 4),
        "ms_per_step_p10_p90": [round(float(np.percentile(step_ms[warm], 10)), 4),
                                round(float(np.percentile(step_ms[warm], 90)), 4)],
        "us_per_layer_step": round(ms / nL * 1e3, 2),
        "step": "per layer: selection + pool update (one launch), then the attention with the gather folded in",
        "ms_per_step_gather_on_side_stream": round(ms_side, 4),
        "ms_per_step_gather_on_side_stream_select_and_update_as_two_launches": round(ms_two, 4),
        "cold_step_ms": round(float(step_ms[0]), 3),
        "hbm_gbps": round(hbm_gbps, 1), "hbm_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "misses_per_unit_layer_step": round(float(n_miss[warm].mean()), 3),
        "miss_fraction": round(float(n_miss[warm].sum() / n_sel[warm].sum()), 4),
        "locality_gamma": round(gamma, 4),
        "host_link_gbps": round(link, 2), "cold_step_host_link_gbps": round(cold_link, 2),
        "memcpy_h2d_gbps": round(link_ref, 2), "host_link_frac_of_memcpy": round(link / link_ref, 4),
        "cold_frac_of_memcpy": round(cold_link / link_ref, 4),
        "gather_share_of_step": round(fetch_share, 4),
        "setup_seconds": round(setup_s, 1),
    }


def _prefill_leg(torch, NI, R, nb):
    """The prefill128k workload: pool the compressed keys and eviction scores of
    a 131072-token prompt, then select for the 64 query rows at its end (each
    row a decode selection at its own position) and attend; then the same
    with one selection shared by the 64 rows.  All timed cold: a 1 GiB
    scratch buffer is streamed before every timed launch, so neither the keys
    (64 MiB) nor the compressed keys (4 MiB) sit in the 256 MB Infinity Cache."""
    w = NI.WORKLOADS["prefill128k"]
    t0 = time.perf_counter()
    K, V, lam, q = NI.layer_inputs(w)
    log(f"inputs {w.name}: {time.perf_counter() - t0:.1f}s")
    kv, logits, qd, pos = _device_inputs(w, K, V, lam, q, R)
    del K, V
    NB = w.n_blocks
    layer = R.DecodeLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, NB, w.dtype, w.kq, w.ke)
    n_q = w.n_steps
    qrows = qd.permute(1, 0, 2, 3).contiguous()             # [B, n_query, Hq, D]
    posr = pos.t().contiguous()                             # [B, n_query]
    sel = torch.full((w.batch, n_q, w.n_kv_heads, w.kq + w.ke), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, n_q, w.n_kv_heads), dtype=torch.int32, device="cuda")
    ws = torch.zeros(nb.workspace_size(layer.dims, nb.OP_SELECT, n_q, w.kq, w.ke), dtype=torch.uint8,
                     device="cuda")
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")    # 1 GiB
    sink = torch.zeros((), dtype=torch.float32, device="cuda")

    def timed(fn, reps=20):
        out = []
        for _ in range(reps):
            sink.copy_(scratch.sum())                           # read 1 GiB: clean, cold caches
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            out.append(a.elapsed_time(b) * 1e3)
        return float(np.median(out)), float(np.percentile(out, 10)), float(np.percentile(out, 90))

    n_tok = w.prompt_len
    units = w.batch * w.n_kv_heads
    complete = n_tok // 64
    pool_us, pool_p10, pool_p90 = timed(lambda: layer.pool_blocks(kv, logits, 0, complete))
    D = w.head_dim
    pool_bytes = units * complete * (64 * D * 2 + 64 * 4 + 4 * D * 2 + 4 * 4 + 4)
    sel_us, sel_p10, sel_p90 = timed(lambda: nb.select_blocks(layer.dims, qrows, n_q, posr, layer.k_comp,
                                                                layer.e_blk, w.kq, w.ke, sel, n_sel, ws))
    c = int(w.positions()[0]) // 64
    G = w.n_q_heads // w.n_kv_heads
    sel_bytes = units * (n_q * 2 * G * D * 2 + 4 * c * D * 2 + 4 * c)
    # exact attention of the 64 rows, each over its own selection and window
    k_cap = w.kq + w.ke
    out = torch.zeros((w.batch, n_q, w.n_q_heads, D), dtype=torch.bfloat16, device="cuda")
    wsa = torch.zeros(nb.workspace_size(layer.dims, nb.OP_ATTN, n_q, k_cap, 0), dtype=torch.uint8, device="cuda")
    attn_us, attn_p10, attn_p90 = timed(lambda: nb.sparse_chunk_attn(layer.dims, qrows, n_q, kv, sel, n_sel, k_cap,
                                                                     posr, None, out, wsa))
    torch.cuda.synchronize()
    # HBM bytes the method must move: every distinct selected block of a KV
    # head once (the rows' selections overlap: Gamma_e is shared), the window
    # blocks, q and out; per-row bytes count each row's blocks separately
    sel_h, n_h = sel.cpu().numpy(), n_sel.cpu().numpy()
    blk_bytes = 64 * 2 * D * 2
    distinct = 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            ids = set()
            for r in range(n_q):
                ids.update(int(x) for x in sel_h[b, r, h, : n_h[b, r, h]])
            distinct += len(ids)
    windows = units * len({int(p) // 64 for p in w.positions()}) * blk_bytes
    qo = units * n_q * 2 * G * D * 2
    attn_bytes = distinct * blk_bytes + windows + qo
    attn_row_bytes = int(n_h.sum()) * blk_bytes + units * n_q * blk_bytes + qo
    log(f"prefill: pooling {pool_us:.1f} us ({pool_bytes / pool_us / 1e3:.0f} GB/s), "
        f"selection of {n_q} rows {sel_us:.1f} us, their attention {attn_us:.1f} us "
        f"({attn_bytes / attn_us / 1e3:.0f} GB/s of distinct blocks)")
    # the chunk-shared variant: one selection for the 64 rows, each row then
    # attends it plus its window
    sh_us, sh_p10, sh_p90 = timed(lambda: nb.select_blocks_shared(layer.dims, qrows, n_q, posr, layer.k_comp,
                                                                  layer.e_blk, w.kq, w.ke, sel, n_sel, ws))
    sha_us, sha_p10, sha_p90 = timed(lambda: nb.sparse_chunk_attn(layer.dims, qrows, n_q, kv, sel, n_sel, k_cap,
                                                                  posr, None, out, wsa))
    torch.cuda.synchronize()
    n_sh = n_sel.cpu().numpy()[:, 0, :]                       # one set per (b, h)
    sha_bytes = int(n_sh.sum()) * blk_bytes + windows + qo
    log(f"prefill, chunk-shared selection: selection {sh_us:.1f} us, attention {sha_us:.1f} us "
        f"({sha_bytes / sha_us / 1e3:.0f} GB/s, {int(n_sh.sum())} blocks)")
    return {
        "workload": "prefill128k", "prompt": n_tok, "query_rows": n_q, "timing": "cold (1 GiB streamed first)",
        "pool_us": round(pool_us, 2), "pool_us_p10_p90": [round(pool_p10, 2), round(pool_p90, 2)],
        "pool_bytes": int(pool_bytes), "pool_gbps": round(pool_bytes / pool_us / 1e3, 1),
        "pool_frac": round(pool_bytes / pool_us / 1e3 / HBM_PEAK_GBPS, 4),
        "select_us": round(sel_us, 2), "select_us_p10_p90": [round(sel_p10, 2), round(sel_p90, 2)],
        "select_bytes": int(sel_bytes),
        "attn_us": round(attn_us, 2), "attn_us_p10_p90": [round(attn_p10, 2), round(attn_p90, 2)],
        "attn_bytes": int(attn_bytes), "attn_gbps": round(attn_bytes / attn_us / 1e3, 1),
        "attn_frac": round(attn_bytes / attn_us / 1e3 / HBM_PEAK_GBPS, 4),
        "attn_row_bytes": int(attn_row_bytes), "attn_distinct_blocks": distinct,
        "shared": {"select_us": round(sh_us, 2), "select_us_p10_p90": [round(sh_p10, 2), round(sh_p90, 2)],
                   "attn_us": round(sha_us, 2), "attn_us_p10_p90": [round(sha_p10, 2), round(sha_p90, 2)],
                   "attn_bytes": sha_bytes, "attn_gbps": round(sha_bytes / sha_us / 1e3, 1),
                   "blocks": int(n_sh.sum())},
    }


def _split_leg(torch, nb):
    """The QKV split with the fused eviction head (nosa_split_qkv), heads as
    layer32k (16 query / 2 KV heads, D = 128, bf16, eviction hidden size 128):
    one decode step (8 batch entries x 1 token, graph of 64 launches) and a
    4096-token chunk of one sequence.  Synthetic rows and weights."""
    Hq, Hkv, D, De, NB = 16, 2, 128, 128, 513
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    w1 = torch.randn((Hkv, D, De), device="cuda", generator=gen) / math.sqrt(D)
    w2 = torch.randn((Hkv, De), device="cuda", generator=gen)
    row = (Hq + 2 * Hkv) * D
    per_tok = row * 2 + Hq * D * 2 + 2 * Hkv * D * 2 + Hkv * 4     # read the row, write q, k, v, logit

    def run(B, n_tok, graph_reps):
        d = nb.dims(B, Hq, Hkv, D, NB, "bf16")
        qkv = torch.randn((B, n_tok, row), device="cuda", generator=gen).to(torch.bfloat16)
        pos = (torch.arange(n_tok, device="cuda", dtype=torch.int32)[None, :] + 64 * 400).repeat(B, 1)
        q_out = torch.empty((B, n_tok, Hq, D), dtype=torch.bfloat16, device="cuda")
        kv = torch.zeros((B, Hkv, NB, 2 * 64 * D), dtype=torch.bfloat16, device="cuda")
        lg = torch.zeros((B, Hkv, NB * 64), dtype=torch.float32, device="cuda")
        call = lambda st=None: nb.split_qkv(d, qkv, n_tok, pos, w1, w2, De, q_out, kv, lg, stream=st)
        call()
        torch.cuda.synchronize()
        st = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for _ in range(graph_reps):
                    call(st)
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(st):
                a.record()
                g.replay()
                b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / graph_reps)
        return float(np.median(ts))

    dec_us = run(8, 1, 64)
    n_chunk = 4096
    chunk_us = run(1, n_chunk, 8)
    chunk_bytes = n_chunk * per_tok + Hkv * D * De * 4 + Hkv * De * 4
    log(f"split_qkv: decode step (8 tokens) {dec_us:.2f} us; {n_chunk}-token chunk {chunk_us:.1f} us "
        f"({chunk_bytes / chunk_us / 1e3:.0f} GB/s)")
    return {
        "heads": [Hq, Hkv], "head_dim": D, "evict_hidden": De, "data": "synthetic rows and weights",
        "decode_tokens": 8, "decode_us": round(dec_us, 2), "decode_bytes": 8 * per_tok + Hkv * D * De * 4,
        "chunk_tokens": n_chunk, "chunk_us": round(chunk_us, 2), "chunk_bytes": int(chunk_bytes),
        "chunk_gbps": round(chunk_bytes / chunk_us / 1e3, 1),
        "chunk_evict_tflops": round(n_chunk * Hkv * D * De * 2 / chunk_us / 1e6, 3),
    }


# The oracle's inputs for the CPU baseline's worker processes (set before the
# pool forks them, so the children share them copy-on-write).
_CPU_ARGS = {}


def _cpu_unit_pass(unit):
    """One pass of the oracle over one (b, h) unit: every decode step."""
    from oracle import nosa_oracle as O
    w, K, V, lam, q = (_CPU_ARGS[k] for k in ("w", "K", "V", "lam", "q"))
    b, h = unit
    G = w.group
    O.decode_unit(K[b, h], V[b, h], lam[b, h], q[:, b, h * G:(h + 1) * G], w.positions(), w.kq, w.ke, bf16=True)
    return 1


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        _CPU_ARGS["limiter"] = threadpool_limits(limits=1)   # one BLAS thread per worker
    except ImportError:                      # pragma: no cover
        pass


def _cpu_baseline(NI, w, K, V, lam, q, min_seconds: float = 10.0, max_passes: int = 400,
                  one_core_seconds: float = 4.0):
    """The oracle, as it stands, on the headline workload, timed on the host
    cores this process may use: the batch's independent (b, h) units spread
    over that many worker processes (forked before the GPU is touched), whole
    passes over every unit and step repeated until about min_seconds.  A
    shorter single-process run on one core is reported beside it."""
    import multiprocessing as mp
    from oracle import nosa_oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover
        threadpool_limits = None
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:                   # pragma: no cover
        host_cores = os.cpu_count() or 1
    units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    G = w.group

    # one core, one process
    limiter = threadpool_limits(limits=1) if threadpool_limits else None
    passes1, t0 = 0, time.perf_counter()
    while True:
        for b, h in units:
            O.decode_unit(K[b, h], V[b, h], lam[b, h], q[:, b, h * G:(h + 1) * G], w.positions(),
                          w.kq, w.ke, bf16=True)
        passes1 += 1
        dt1 = time.perf_counter() - t0
        if dt1 >= one_core_seconds or passes1 >= max_passes:
            break
    if limiter is not None:
        limiter.restore_original_limits()
    one_core = passes1 * w.batch * w.n_steps / dt1

    # every host core: units spread over the worker processes
    n_proc = max(1, min(len(units), host_cores))
    _CPU_ARGS.update(w=w, K=K, V=V, lam=lam, q=q)
    ctx = mp.get_context("fork")
    with ctx.Pool(n_proc, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_unit_pass, units)      # workers started and warm (untimed)
        passes, t0 = 0, time.perf_counter()
        while True:
            pool.map(_cpu_unit_pass, units, chunksize=1)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds or passes >= max_passes:
                break
    _CPU_ARGS.clear()
    tokens = passes * w.batch * w.n_steps
    n_pass = f"{passes} pass" + ("" if passes == 1 else "es")
    log(f"oracle: {tokens} tokens ({n_pass}) in {dt:.1f}s on {n_proc} processes; one core "
        f"{one_core:.0f} tokens/s")
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": n_proc, "host_cores": host_cores,
            "kind": "oracle", "one_core_value": round(one_core, 3),
            "sample": f"the whole layer32k workload, {n_pass}: {len(units)} (batch entry, KV head) units, all "
                      f"{w.n_steps} decode steps each, incl. pooling the 32K prompt; numpy with BLAS limited to one "
                      f"thread per process, the units spread over {n_proc} forked processes (the host cores this "
                      f"process may use: {host_cores}); one_core_value: the same passes in one process",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
