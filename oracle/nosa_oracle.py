"""CPU oracle of the NOSA decode path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does,
and this module imports nothing from the library.  It shares no code with the
HIP kernels: the only shared module is the seeded input generator.

Sources (the web pages describing NOSA, arXiv 2510.13602):

* montaan.com summary "NOSA: Native and Offloadable Sparse Attention",
  sections "How it works" (Eq. 3, two Top-k functions), "Key Design
  Components" items 1-4 (eviction rule, two-stage block pooling, Eq. 4, Eq. 7)
  and "System Optimization (NOSI)" item 2 (block-sized units, swap only the
  blocks unused this step).
* gist.science summary "Résumé Technique : NOSA", section "1. Algorithme :
  NOSA" (dual selection, locality guarantee gamma(t) >= ke/k, mean pooling
  within sub-blocks then max pooling per block, ED-DMA pre-exponential
  selection) and "2. Système : NOSI" (set differences for block swapping).
* wmrh.cn NOSA-1B release post, sections "NOSA-1B 是什么" (only the current
  window and the Top-K blocks stay on the GPU) and "工程实现亮点" (two-stage
  attention: compressed KV picks Top-K blocks, then exact attention; block
  size and Top-K both 64).

Readings taken where the pages leave a step open:

* U1  Eq. 7: Gamma = Gamma_q U Gamma_e, two independent top-k sets.
* U2  scores, not keys, are max-pooled: sigma per 16-token sub-block mean,
      block score = max over its 4 sub-blocks.
* U3  GQA: one selection per KV head, query = sum of its G query heads.
* U4  selection is on raw dot products: no 1/sqrt(D), no exp, no softmax.
* U5  eviction logits are an input per (batch, KV head, token), fp32.
* U6  no eviction bias inside the attention.
* U7  window = the current (partial) block, always attended, not counted in k.
* U8  decode step t sits at p = L + t and attends tokens [0, p].
* U9  ties ordered by (score descending, block id ascending).
* U10 fewer candidates than budget: take them all.
* U11 pooled keys: fp32 left-to-right sum of the 16 tokens, x 0.0625, one
      round-to-nearest-even to bf16 (kept fp32 for fp32 workloads).  The same
      for the logits (kept fp32).  This decides a quantised value, so it is
      taken in the precision the kernels use (fp32), not fp64.
* U12 attention: scale 1/sqrt(D), softmax over the selected blocks plus the
      window, computed in float64, output rounded once.
* U13 pool: each miss (ascending id) takes the lowest free slot, else evicts
      the resident block not needed this step with the smallest
      (last_use, block id); a block completed by the window is inserted first
      with last_use = t - 1 under the same rule (nothing happens when it is
      already resident).  If a miss of the same step evicts the inserted
      block again, no insertion is reported (insert_slot = -1): the window
      block must not be copied over the slot the miss now owns.
* U14 gamma(t) counted in blocks, window of t-1 counted as held at t-1.
* U16 several query rows: each row is a decode selection at its own position.
* U19 eviction head (Eq. 4): per KV head, W1 is D x De and W2 has De
      entries (the pages give no shapes; De is a parameter), tau = softplus
      log(1 + e^x); weights fp32; computed here in float64.
* U20 chunk-shared selection (a variant of U16): one selection for all
      rows of a prefill chunk, scored with the sum over the rows of their
      summed query heads (U3 applied to the whole chunk); the candidates are
      the complete blocks before the first row's block; every row attends the
      shared set plus its own window.

Alternative readings, each behind a flag and off by default (the library's
own path follows U1 and U6):

* U21 Eq. 7 read as "fill the remainder from the candidates left": the
      query-agnostic part is the top-ke of E over the candidates outside
      Gamma_q, so the union holds exactly min(kq + ke, c) blocks.  A block can
      then leave the query-agnostic part and come back later, which the
      eviction rule forbids (montaan "Key Design Components" items 1, 4).
* U22 ED-DMA's deferred exponential read as an additive logit: the eviction
      score of each attended token (its pre-exponential logit, U5) is added to
      that token's attention logit, softmax(q K^T / sqrt(D) + lambda)
      (gist.science "1. Algorithme : NOSA", the ED-DMA item: the exponential
      is applied at the attention step).

Pins: every function here is pinned by a test against something other than
itself (a library routine, brute force, a closed form or a stated invariant);
none is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 64
SUB = 16
SUBS_PER_BLOCK = BLOCK // SUB


# --------------------------------------------------------------------------
# rounding of stored values
# --------------------------------------------------------------------------
def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value, ties to even; result held as float32.

    Written from the definition: keep the top 16 bits of the float32 pattern,
    rounding on the 16 dropped bits.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.int64)
    lower = bits & 0xFFFF
    upper = bits >> 16
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    upper = upper + round_up.astype(np.int64)
    return (upper.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


# --------------------------------------------------------------------------
# O1-O3: compressed keys and the compressed informative score (CIS)
# (gist.science "Implémentation par blocs": mean pooling within sub-blocks,
#  then max pooling per block, for the selection scores of both selections;
#  montaan "Key Design Components" item 2.)
# --------------------------------------------------------------------------
def subblock_key_means(K: np.ndarray, bf16: bool) -> np.ndarray:
    """Mean of every complete 16-token sub-block of K [T, D].

    fp32 additions strictly in token order, then x 1/16 (exact), then one
    rounding to bf16 if the workload is bf16 (reading U11).
    """
    K = np.asarray(K, dtype=np.float32)
    n_sub = K.shape[0] // SUB
    rows = K[: n_sub * SUB].reshape(n_sub, SUB, K.shape[1])
    acc = rows[:, 0, :].copy()
    for i in range(1, SUB):
        acc = acc + rows[:, i, :]          # float32 + float32, token order
    mean = acc * np.float32(0.0625)
    return to_bf16(mean) if bf16 else mean


def subblock_logit_means(lam: np.ndarray) -> np.ndarray:
    """Mean of the eviction logits of every complete 16-token sub-block (fp32)."""
    lam = np.asarray(lam, dtype=np.float32)
    n_sub = lam.shape[0] // SUB
    rows = lam[: n_sub * SUB].reshape(n_sub, SUB)
    acc = rows[:, 0].copy()
    for i in range(1, SUB):
        acc = acc + rows[:, i]
    return acc * np.float32(0.0625)


def block_eviction_scores(e_sub: np.ndarray) -> np.ndarray:
    """Block score E_b = max of the means of its 4 sub-blocks (complete blocks)."""
    n_blk = e_sub.shape[0] // SUBS_PER_BLOCK
    out = np.empty(n_blk, dtype=np.float32)
    for b in range(n_blk):
        out[b] = max(e_sub[SUBS_PER_BLOCK * b + i] for i in range(SUBS_PER_BLOCK))
    return out


# --------------------------------------------------------------------------
# O5: query-aware block scores (montaan "How it works": a Top-k over the
# query's scores; gist.science ED-DMA: select on pre-exponential scores)
# --------------------------------------------------------------------------
def query_block_scores(q_group: np.ndarray, kbar: np.ndarray, n_cand: int) -> np.ndarray:
    """Score of each candidate block 0..n_cand-1 for one KV head.

    q_group: [G, D] the query heads sharing the KV head; kbar: [>=4*n_cand, D].
    sigma_j = (sum_g q_g) . kbar_j in float64; block score = max over its 4
    sub-blocks (readings U2, U3, U4).
    """
    qsum = np.asarray(q_group, dtype=np.float64).sum(axis=0)
    sig = np.asarray(kbar[: SUBS_PER_BLOCK * n_cand], dtype=np.float64) @ qsum
    out = np.empty(n_cand, dtype=np.float64)
    for b in range(n_cand):
        out[b] = max(sig[SUBS_PER_BLOCK * b + i] for i in range(SUBS_PER_BLOCK))
    return out


# --------------------------------------------------------------------------
# O6: selection, Eq. 7 (montaan "Key Design Components" item 4)
# --------------------------------------------------------------------------
def top_blocks(scores: Sequence[float], budget: int) -> List[int]:
    """Ids of the `budget` best candidates by (score desc, id asc) (U9, U10)."""
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return order[: max(0, min(budget, len(scores)))]


def select_blocks(s_q: Sequence[float], E: Sequence[float], n_cand: int,
                  kq: int, ke: int) -> Tuple[List[int], List[int], List[int]]:
    """Gamma_q, Gamma_e and their union (ascending) over candidates 0..n_cand-1."""
    g_q = top_blocks(list(s_q[:n_cand]), kq)
    g_e = top_blocks(list(E[:n_cand]), ke)
    return sorted(g_q), sorted(g_e), sorted(set(g_q) | set(g_e))


def select_blocks_fill(s_q: Sequence[float], E: Sequence[float], n_cand: int,
                       kq: int, ke: int) -> Tuple[List[int], List[int], List[int]]:
    """Eq. 7 read as U21: Gamma_q as in select_blocks, then the query-agnostic
    part is the top-ke of E over the candidates not in Gamma_q.  Returns
    (Gamma_q, the query-agnostic part, their union), each ascending."""
    g_q = top_blocks(list(s_q[:n_cand]), kq)
    in_q = set(g_q)
    rest = [j for j in range(n_cand) if j not in in_q]
    g_e = [rest[i] for i in top_blocks([E[j] for j in rest], ke)]
    return sorted(g_q), sorted(g_e), sorted(in_q | set(g_e))


def chunk_shared_selection(q_rows: np.ndarray, first_pos: int, kbar: np.ndarray, E: Sequence[float],
                           kq: int, ke: int) -> Tuple[List[int], List[int], List[int]]:
    """One Eq. 7 selection for all rows of a prefill chunk (reading U20).

    q_rows: [n_query, G, D] the chunk's query heads of one KV head; first_pos:
    the first row's position (its block bounds the candidates; a negative
    position leaves none).  The chunk is one query group: its score is
    query_block_scores over every row's heads together.
    """
    q_rows = np.asarray(q_rows)
    n_cand = first_pos // BLOCK if first_pos >= 0 else 0
    s_q = query_block_scores(q_rows.reshape(-1, q_rows.shape[-1]), kbar, n_cand)
    return select_blocks(s_q, E, n_cand, kq, ke)


# --------------------------------------------------------------------------
# The eviction head of Eq. 4 (montaan summary, "Key Design Components" item 3:
# s^e_j = tau(v_j W1) W2 with tau the softplus of DMA's design), one KV head;
# its scores are the logits that O2 pools.
# --------------------------------------------------------------------------
def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x), without overflow."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def eviction_logits(V: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """V [T, D], W1 [D, De], W2 [De] -> s^e [T] (float64)."""
    h = np.asarray(V, dtype=np.float64) @ np.asarray(W1, dtype=np.float64)
    return softplus(h) @ np.asarray(W2, dtype=np.float64)


# --------------------------------------------------------------------------
# O7: exact attention over the selected blocks plus the window
# (wmrh.cn "工程实现亮点": the selected blocks get exact attention)
# --------------------------------------------------------------------------
def attended_tokens(S: Sequence[int], pos: int) -> np.ndarray:
    c = pos // BLOCK
    toks = [np.arange(BLOCK * b, BLOCK * b + BLOCK) for b in sorted(S)]
    toks.append(np.arange(BLOCK * c, pos + 1))
    return np.concatenate(toks)


def sparse_attention(q_group: np.ndarray, K: np.ndarray, V: np.ndarray,
                     S: Sequence[int], pos: int, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """o_g = softmax(q_g K_T^T / sqrt(D) [+ bias_T]) V_T for T = selected blocks + window.

    bias (reading U22): per-token additive logits [>= pos + 1], natural-log
    units, the same for every query head.  float64 throughout; returns [G, D]
    float64 (the caller rounds).
    """
    idx = attended_tokens(S, pos)
    q = np.asarray(q_group, dtype=np.float64)
    k = np.asarray(K[idx], dtype=np.float64)
    v = np.asarray(V[idx], dtype=np.float64)
    logits = (q @ k.T) / math.sqrt(q.shape[1])
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[idx][None, :]
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ v


def round_output(o: np.ndarray, bf16: bool) -> np.ndarray:
    return to_bf16(o.astype(np.float32)) if bf16 else o.astype(np.float32)


# --------------------------------------------------------------------------
# O8: HBM block pool bookkeeping (montaan "System Optimization (NOSI)" item 2;
# gist.science "2. Système : NOSI": set differences for block swapping)
# --------------------------------------------------------------------------
@dataclass
class BlockPool:
    n_slots: int
    slot_block: List[int] = field(default_factory=list)
    slot_last_use: List[int] = field(default_factory=list)

    def __post_init__(self):
        self.slot_block = [-1] * self.n_slots
        self.slot_last_use = [-1] * self.n_slots

    def slot_of(self, block: int) -> int:
        for s, b in enumerate(self.slot_block):
            if b == block:
                return s
        return -1

    def resident(self) -> set:
        return {b for b in self.slot_block if b >= 0}

    def _take_slot(self, needed: set) -> int:
        for s in range(self.n_slots):          # lowest free slot first
            if self.slot_block[s] < 0:
                return s
        best = None
        for s in range(self.n_slots):          # else least recently used block not needed now
            b = self.slot_block[s]
            if b in needed:
                continue
            key = (self.slot_last_use[s], b)
            if best is None or key < best[0]:
                best = (key, s)
        if best is None:
            raise RuntimeError("pool too small for the blocks needed this step")
        return best[1]

    def step(self, t: int, S: Sequence[int], insert: Optional[int] = None):
        """One step of the pool.  Returns (misses [(block, slot)], insert_slot, phys).

        `insert` is a block that the window just completed (held in HBM); it is
        placed first, with last_use = t - 1, and is not a host fetch.
        insert_slot is the slot it holds at the end of the step (-1 if there
        was no insertion or a miss of the same step evicted it again).
        """
        needed = set(S)
        insert_slot = -1
        if insert is not None and insert >= 0 and self.slot_of(insert) < 0:
            insert_slot = self._take_slot(needed)
            self.slot_block[insert_slot] = insert
            self.slot_last_use[insert_slot] = t - 1
        misses = []
        for b in sorted(needed - self.resident()):
            s = self._take_slot(needed)
            self.slot_block[s] = b
            misses.append((b, s))
        if insert_slot >= 0 and self.slot_block[insert_slot] != insert:
            insert_slot = -1                   # placed, then evicted again this step
        phys = []
        for b in sorted(needed):
            s = self.slot_of(b)
            self.slot_last_use[s] = t
            phys.append(s)
        return misses, insert_slot, phys


# --------------------------------------------------------------------------
# O9: locality (montaan "How it works", Eq. 3; gist.science "Garantie de
# localité": gamma(t) >= ke/k)
# --------------------------------------------------------------------------
def readmissions(gamma_e: Sequence[Sequence[int]]) -> int:
    """Blocks that re-enter the query-agnostic part after leaving it, summed
    over the steps: the eviction rule (montaan "Key Design Components"
    item 1) says this is 0."""
    dropped, count = set(), 0
    for t in range(len(gamma_e)):
        cur = set(gamma_e[t])
        count += len(cur & dropped)
        if t > 0:
            dropped |= set(gamma_e[t - 1]) - cur
        dropped -= cur
    return count


def locality(S_prev: Sequence[int], window_prev: int, S: Sequence[int]) -> float:
    if len(S) == 0:
        return 1.0
    held = set(S_prev) | {window_prev}
    return len(set(S) & held) / len(S)


# --------------------------------------------------------------------------
# whole decode loop of one (batch, KV head) unit
# --------------------------------------------------------------------------
@dataclass
class UnitTrace:
    sel: List[List[int]] = field(default_factory=list)
    gamma_q: List[List[int]] = field(default_factory=list)
    gamma_e: List[List[int]] = field(default_factory=list)
    s_q: List[np.ndarray] = field(default_factory=list)
    out: List[np.ndarray] = field(default_factory=list)       # [G, D] rounded
    misses: List[List[Tuple[int, int]]] = field(default_factory=list)
    insert_slot: List[int] = field(default_factory=list)
    phys: List[List[int]] = field(default_factory=list)
    locality: List[float] = field(default_factory=list)


def decode_unit(K: np.ndarray, V: np.ndarray, lam: np.ndarray, q_rows: np.ndarray,
                positions: Sequence[int], kq: int, ke: int, bf16: bool,
                pool_slots: Optional[int] = None, attend: bool = True,
                forced_sel: Optional[Dict[int, List[int]]] = None,
                fill_remaining: bool = False, evict_bias: bool = False,
                pool_reset_at: Optional[int] = None) -> UnitTrace:
    """Run the path for one (batch, KV head) over consecutive decode positions.

    K, V: [T, D]; lam: [T]; q_rows: [n, G, D]; positions: the n positions.
    `forced_sel` maps a step to a selection to use in place of the oracle's
    own (used to keep lock-step when a score tie is accepted).
    `fill_remaining` selects with reading U21 (gamma_e then holds the
    query-agnostic part), `evict_bias` attends with reading U22.
    `pool_reset_at`: at that step the pool starts again empty (a restart that
    forgets every resident block; the selection is not affected).
    """
    kbar = subblock_key_means(K, bf16)
    E = block_eviction_scores(subblock_logit_means(lam))
    pool = BlockPool(pool_slots) if pool_slots else None
    tr = UnitTrace()
    prev_S: Optional[List[int]] = None
    prev_c: Optional[int] = None
    for t, p in enumerate(positions):
        c = int(p) // BLOCK
        s_q = query_block_scores(q_rows[t], kbar, c)
        pick = select_blocks_fill if fill_remaining else select_blocks
        g_q, g_e, S = pick(s_q, E, c, kq, ke)
        if forced_sel is not None and t in forced_sel:
            S = sorted(forced_sel[t])
        tr.s_q.append(s_q)
        tr.gamma_q.append(g_q)
        tr.gamma_e.append(g_e)
        tr.sel.append(S)
        if pool is not None:
            if t == pool_reset_at:
                pool = BlockPool(pool_slots)
            insert = prev_c if (prev_c is not None and c > prev_c) else None
            misses, ins_slot, phys = pool.step(t, S, insert)
            tr.misses.append(misses)
            tr.insert_slot.append(ins_slot)
            tr.phys.append(phys)
        if attend:
            tr.out.append(round_output(sparse_attention(q_rows[t], K, V, S, int(p), lam if evict_bias else None),
                                       bf16))
        tr.locality.append(locality(prev_S, prev_c, S) if prev_S is not None else float("nan"))
        prev_S, prev_c = S, c
    return tr
