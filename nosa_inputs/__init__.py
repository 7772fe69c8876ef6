"""Seeded synthetic inputs for the NOSA decode path.

This module holds only shapes, seeds and random draws.  It contains none of
the method's arithmetic (no pooling, scoring, selection or attention), so both
the CPU oracle and the HIP path may take their inputs from it.

Workloads (the long-context decode settings of "NOSA: Native and Offloadable
Sparse Attention", montaan summary, "Empirical Results"; the 1B model shape of
the wmrh.cn NOSA-1B release post: 16 heads, bf16, 64-token blocks, top-64):

* ``tiny``     1 layer, B=1, 2 query heads / 1 KV head, D=64, context 4096,
               kq=4, ke=4, fp32, 16 decode steps, i.i.d. N(0,1) queries.
* ``layer32k`` B=8, 16/2 heads, D=128, context 32768, kq=16, ke=48, bf16,
               64 decode steps, AR(1) queries (rho = 0.9).
* ``offload``  heads as ``layer32k``, B=64, context 16384, HBM pool of 80
               blocks per KV head, 128 steps, KV in pinned host memory.
* ``stack128k`` 28 layers of ``layer32k`` attention, B=16, context 131072,
               pool of 80, 32 steps.
* ``prefill128k`` B=1, 16/2 heads, D=128, prompt 131072, selection for the
               64 query rows at the end of the prompt.

Recipe (identical for every workload):

* seed = 20251015 + 100 * config_index + layer; a numpy PCG64 stream.
* stream 0 draws the queries; stream u+1 (``PCG64.jumped(u+1)``) draws the
  (batch b, KV head h) unit u = b*Hkv + h, so any unit can be regenerated
  alone.  Within a unit the draw order is: per-block key offsets mu
  (NB x D, std 0.5), key noise (T x D), values (T x D), eviction logits (T).
* K = N(0,1) + mu[block of the token]; V = N(0,1); logits = N(0,1) (fp32).
* queries: q_0 ~ N(0,1); q_t = rho*q_{t-1} + sqrt(1-rho^2)*eps_t, drawn per
  step in the order [B, Hq, D].  rho = 0 gives i.i.d. queries.
* values are drawn in fp32 and, for bf16 workloads, rounded to the nearest
  bf16 (ties to even); they are returned as float32 arrays holding exactly
  representable bf16 values.  The eviction logits stay fp32.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

BLOCK = 64      # tokens per KV block
SUB = 16        # tokens per sub-block of the compressed keys
BASE_SEED = 20251015


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the workload list; enters the seed
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prompt_len: int       # L: positions 0..L-1 form the prompt
    n_steps: int          # decode steps (or query rows for prefill128k)
    kq: int
    ke: int
    dtype: str            # "bf16" or "f32"
    rho: float            # AR(1) coefficient of the queries
    pool_slots: Optional[int] = None   # HBM pool blocks per KV head (offload)
    n_layers: int = 1
    prefill: bool = False              # queries sit at the end of the prompt

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def total_tokens(self) -> int:
        """Positions that hold keys: the prompt plus every decode step."""
        return self.prompt_len if self.prefill else self.prompt_len + self.n_steps

    @property
    def n_blocks(self) -> int:
        return math.ceil(self.total_tokens / BLOCK)

    def positions(self) -> np.ndarray:
        """Position of each query row (decode step t sits at L + t)."""
        if self.prefill:
            return np.arange(self.prompt_len - self.n_steps, self.prompt_len, dtype=np.int64)
        return np.arange(self.prompt_len, self.prompt_len + self.n_steps, dtype=np.int64)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 2, 1, 64, 4096, 16, 4, 4, "f32", 0.0),
    "layer32k": Workload("layer32k", 1, 8, 16, 2, 128, 32768, 64, 16, 48, "bf16", 0.9),
    "offload": Workload("offload", 2, 64, 16, 2, 128, 16384, 128, 16, 48, "bf16", 0.9, pool_slots=80),
    "stack128k": Workload("stack128k", 3, 16, 16, 2, 128, 131072, 32, 16, 48, "bf16", 0.9,
                          pool_slots=80, n_layers=28),
    "prefill128k": Workload("prefill128k", 4, 1, 16, 2, 128, 131072, 64, 16, 48, "bf16", 0.9,
                            prefill=True),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (small test cases)."""
    return dataclasses.replace(w, **changes)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & 1          # ties go to the even neighbour
    r += 0x7FFF
    r += u                     # no wrap for finite inputs: at most 0xFF807FFF
    r &= 0xFFFF0000
    return r.view(np.float32)


def _seed(w: Workload, layer: int) -> int:
    return BASE_SEED + 100 * w.index + layer


def _quantise(w: Workload, x: np.ndarray) -> np.ndarray:
    return round_to_bf16(x) if w.dtype == "bf16" else x.astype(np.float32)


def unit_kv(w: Workload, b: int, h: int, layer: int = 0, n_tokens: Optional[int] = None):
    """Keys, values and eviction logits of one (batch, KV head) unit.

    Returns K [T, D], V [T, D] (float32, bf16-valued for bf16 workloads) and
    logits [T] float32, T = ``n_tokens`` (default: the workload's total).
    """
    T = w.total_tokens if n_tokens is None else n_tokens
    nb = math.ceil(T / BLOCK)
    bg = np.random.PCG64(_seed(w, layer)).jumped(1 + b * w.n_kv_heads + h)
    rng = np.random.Generator(bg)
    D = w.head_dim
    mu = rng.standard_normal((nb, D), dtype=np.float32) * np.float32(0.5)
    k = rng.standard_normal((T, D), dtype=np.float32)
    k += np.repeat(mu, BLOCK, axis=0)[:T]
    v = rng.standard_normal((T, D), dtype=np.float32)
    lam = rng.standard_normal(T, dtype=np.float32)
    return _quantise(w, k), _quantise(w, v), lam


def queries(w: Workload, layer: int = 0) -> np.ndarray:
    """Query rows [n_steps, B, Hq, D] (float32, bf16-valued for bf16 workloads)."""
    rng = np.random.Generator(np.random.PCG64(_seed(w, layer)))
    shape = (w.batch, w.n_q_heads, w.head_dim)
    q = np.empty((w.n_steps,) + shape, dtype=np.float32)
    cur = rng.standard_normal(shape, dtype=np.float32)
    q[0] = cur
    a = np.float32(w.rho)
    s = np.float32(math.sqrt(max(0.0, 1.0 - w.rho * w.rho)))
    for t in range(1, w.n_steps):
        eps = rng.standard_normal(shape, dtype=np.float32)
        cur = a * cur + s * eps if w.rho != 0.0 else eps
        q[t] = cur
    return _quantise(w, q)


def layer_inputs(w: Workload, layer: int = 0, n_tokens: Optional[int] = None, workers: int = 1):
    """Whole-layer inputs: K, V [B, Hkv, T, D], logits [B, Hkv, T], q [n, B, Hq, D].

    Every (batch, KV head) unit has its own stream, so ``workers`` > 1 draws
    units on that many threads with identical results."""
    T = w.total_tokens if n_tokens is None else n_tokens
    K = np.empty((w.batch, w.n_kv_heads, T, w.head_dim), np.float32)
    V = np.empty_like(K)
    lam = np.empty((w.batch, w.n_kv_heads, T), np.float32)

    def fill(u):
        b, h = divmod(u, w.n_kv_heads)
        K[b, h], V[b, h], lam[b, h] = unit_kv(w, b, h, layer, T)

    units = range(w.batch * w.n_kv_heads)
    if workers > 1:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, units))
    else:
        for u in units:
            fill(u)
    return K, V, lam, queries(w, layer)


def host_workers() -> int:
    """Threads for input generation: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))
