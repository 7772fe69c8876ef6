"""Decode-step driver: device buffers of one attention layer and the order of
the libnosa calls per step.

Two modes:

* resident -- the whole KV cache of the layer sits in HBM; attention reads
  the selected blocks in place (phys = the selected block ids) and the
  window straight from the cache;
* offload  -- the KV cache sits in pinned host memory; a fixed HBM pool of
  `pool_slots` blocks per KV head holds the selected blocks, refilled each
  step (NOSI's design: only the window and the Top-K blocks stay on the GPU,
  the rest is offloaded).

Per step, resident: select, then attention (or both in one launch,
nosa_decode_step).  Offload, on one stream: select, fetch, attention over the
pool; or overlapped, with a side stream: select and the pool update on the
compute stream, then the gather of the misses on the side stream while the
first part of the pool attention (the resident hits and the window) runs on
the compute stream, then the second part (the fetched blocks and the merge)
once both are done.  The compressed keys of a block are built once, when the
block is complete.  All buffers are torch tensors; torch provides device
memory, pinned host memory and streams, and nothing else.  `OffloadStack`
runs several offload layers one after another per decode step.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import binding as nb

BLOCK = nb.BLOCK


def torch_dtype(dtype: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def _fragment_sources(D: int, bf16: bool):
    """(token, dim) read by every element of a block's key half and value half.

    The library stores a block in MFMA fragment order: 1 KiB fragments of
    64 lanes x 16 bytes.  bf16: key fragment (t, s) lane 16g+r holds
    K[tile_token(t, r)][32s+8g .. +7]; value fragment (h, u) lane 16g+r holds
    V[32h+8g .. +7][16u+r]; tile_token(t, r) = 32(t//2) + 8(r//4) + 4(t%2) + r%4.
    fp32: key fragment (t, s) lane 16g+r holds K[16t+r][16s+4g .. +3]; value
    fragment (t, u) lane 16g+r holds V[16t+4g .. +3][16u+r].
    """
    n = BLOCK * D
    p = np.arange(n)
    if bf16:
        nk = D // 32
        j, lane = p % 8, (p // 8) % 64
        g, r = lane // 16, lane % 16
        t, s = p // (nk * 512), (p // 512) % nk
        k_tok = 32 * (t // 2) + 8 * (r // 4) + 4 * (t % 2) + r % 4
        k_dim = 32 * s + 8 * g + j
        nd = D // 16
        h, u = p // (nd * 512), (p // 512) % nd
        v_tok = 32 * h + 8 * g + j
        v_dim = 16 * u + r
    else:
        nk = nd = D // 16
        j, lane = p % 4, (p // 4) % 64
        g, r = lane // 16, lane % 16
        t, s = p // (nk * 256), (p // 256) % nk
        k_tok, k_dim = 16 * t + r, 16 * s + 4 * g + j
        v_tok, v_dim = 16 * t + 4 * g + j, 16 * (p // 256 % nd) + r
    return k_tok * D + k_dim, v_tok * D + v_dim


def pack_kv_blocks(K: torch.Tensor, V: torch.Tensor, n_blocks: int) -> torch.Tensor:
    """Lay K, V [B, Hkv, T, D] out in the library's block format.

    Returns [B, Hkv, n_blocks, 2*64*D]: per block the keys, then the values,
    each in MFMA fragment order (see _fragment_sources).  Tokens past T are
    zero.
    """
    B, H, T, D = K.shape
    pad = n_blocks * BLOCK - T
    if pad < 0:
        raise ValueError("n_blocks too small for T")
    if pad:
        K = torch.nn.functional.pad(K, (0, 0, 0, pad))
        V = torch.nn.functional.pad(V, (0, 0, 0, pad))
    ks, vs = _fragment_sources(D, K.dtype == torch.bfloat16)
    ks = torch.from_numpy(ks).to(K.device)
    vs = torch.from_numpy(vs).to(K.device)
    kb = K.reshape(B, H, n_blocks, BLOCK * D).index_select(-1, ks)
    vb = V.reshape(B, H, n_blocks, BLOCK * D).index_select(-1, vs)
    return torch.cat([kb, vb], dim=-1).contiguous()


def pad_logits(lam: torch.Tensor, n_blocks: int) -> torch.Tensor:
    B, H, T = lam.shape
    out = torch.zeros(B, H, n_blocks * BLOCK, dtype=torch.float32, device=lam.device)
    out[:, :, :T] = lam
    return out


class DecodeLayer:
    """One layer's NOSA decode state on the GPU."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, n_blocks: int,
                 dtype: str, kq: int, ke: int, pool_slots: Optional[int] = None,
                 device: str = "cuda"):
        self.B, self.Hq, self.Hkv, self.D, self.NB = batch, n_q_heads, n_kv_heads, head_dim, n_blocks
        self.dtype, self.kq, self.ke, self.k = dtype, kq, ke, kq + ke
        self.tdt = torch_dtype(dtype)
        self.dev = torch.device(device)
        self.dims = nb.dims(batch, n_q_heads, n_kv_heads, head_dim, n_blocks, dtype)
        self.blk_elems = 2 * BLOCK * head_dim
        self.scale = 1.0 / math.sqrt(head_dim)
        B, H, NB, D = batch, n_kv_heads, n_blocks, head_dim
        z = dict(device=self.dev)
        self.k_comp = torch.zeros(B, H, NB * 4, D, dtype=self.tdt, **z)
        self.e_sub = torch.zeros(B, H, NB * 4, dtype=torch.float32, **z)
        self.e_blk = torch.zeros(B, H, NB, dtype=torch.float32, **z)
        self.sel = torch.full((B, H, max(self.k, 1)), -1, dtype=torch.int32, **z)
        self.n_sel = torch.zeros(B, H, dtype=torch.int32, **z)
        self.out = torch.zeros(B, n_q_heads, D, dtype=self.tdt, **z)
        self.ws_sel = torch.zeros(nb.workspace_size(self.dims, nb.OP_SELECT, 1, kq, ke), dtype=torch.uint8, **z)
        self.ws_attn = torch.zeros(nb.workspace_size(self.dims, nb.OP_ATTN, 1, kq, ke), dtype=torch.uint8, **z)
        self.ws_step = None
        self.pool_slots = pool_slots
        if pool_slots:
            P = pool_slots
            self.pool = torch.zeros(B, H, P, self.blk_elems, dtype=self.tdt, **z)
            self.block_table = torch.full((B, H, NB), -1, dtype=torch.int32, **z)
            self.slot_block = torch.full((B, H, P), -1, dtype=torch.int32, **z)
            self.slot_last_use = torch.full((B, H, P), -1, dtype=torch.int32, **z)
            self.phys = torch.full((B, H, max(self.k, 1)), -1, dtype=torch.int32, **z)
            self.miss_list = torch.full((B, H, self.k + 1, 2), -1, dtype=torch.int32, **z)
            self.n_miss = torch.zeros(B, H, dtype=torch.int32, **z)

    # -- compressed keys ------------------------------------------------
    def pool_blocks(self, kv: torch.Tensor, logits: torch.Tensor, blk_begin: int, blk_end: int,
                    stream=None) -> None:
        """Compressed keys + eviction scores of blocks [blk_begin, blk_end) of the HBM cache."""
        nb.pool_keys(self.dims, kv, self.NB * self.blk_elems, self.blk_elems, logits, blk_begin,
                     blk_end, self.k_comp, self.e_sub, self.e_blk, stream=stream)

    def pool_window(self, window: torch.Tensor, logits: torch.Tensor, block: int, stream=None) -> None:
        """Compressed keys of one completed block held in a window buffer [B, Hkv, block]."""
        nb.pool_keys(self.dims, window, self.blk_elems, 0, logits, block, block + 1, self.k_comp,
                     self.e_sub, self.e_blk, stream=stream)

    def pool_entries(self, kv: torch.Tensor, logits: torch.Tensor, entry_block: torch.Tensor,
                     unit_stride: Optional[int] = None, block_stride: Optional[int] = None, stream=None) -> None:
        """Compressed keys of one block per batch entry (entry_block: device
        int32 [B], -1 for none), read from the HBM cache, or with
        unit_stride = block and block_stride = 0 from a window buffer
        [B, Hkv, block] holding each entry's block."""
        us = self.NB * self.blk_elems if unit_stride is None else unit_stride
        bs = self.blk_elems if block_stride is None else block_stride
        nb.pool_keys_entries(self.dims, kv, us, bs, logits, entry_block, self.k_comp, self.e_sub, self.e_blk,
                             stream=stream)

    # -- one decode step -------------------------------------------------
    def select(self, q: torch.Tensor, pos: torch.Tensor, stream=None, fill: bool = False) -> None:
        """nosa_select_blocks, or with fill=True its variant nosa_select_blocks_fill."""
        call = nb.select_blocks_fill if fill else nb.select_blocks
        call(self.dims, q, 1, pos, self.k_comp, self.e_blk, self.kq, self.ke, self.sel, self.n_sel, self.ws_sel,
             stream=stream)

    def attend_resident_bias(self, q: torch.Tensor, kv: torch.Tensor, pos: torch.Tensor, logits: torch.Tensor,
                             stream=None) -> None:
        """nosa_sparse_decode_attn_bias: the eviction logits added to the attention logits."""
        nb.sparse_decode_attn_bias(self.dims, q, kv, self.sel, self.n_sel, self.k, pos, self.scale, logits,
                                   self.out, self.ws_attn, stream=stream)

    def attend_resident(self, q: torch.Tensor, kv: torch.Tensor, pos: torch.Tensor, stream=None) -> None:
        nb.sparse_decode_attn(self.dims, q, kv, self.NB, self.sel, self.n_sel, self.k, kv,
                              self.NB * self.blk_elems, self.blk_elems, pos, self.scale, self.out,
                              self.ws_attn, stream=stream)

    def fetch(self, host_kv: torch.Tensor, step: int, insert_block: Optional[torch.Tensor] = None,
              insert_src: Optional[torch.Tensor] = None, stream=None) -> None:
        nb.fetch_blocks(self.dims, host_kv, self.pool, self.pool_slots, self.block_table,
                        self.slot_block, self.slot_last_use, step, self.sel, self.n_sel, self.k,
                        insert_block, insert_src, self.phys, self.miss_list, self.n_miss,
                        stream=stream)

    def attend_pool(self, q: torch.Tensor, window: torch.Tensor, pos: torch.Tensor, stream=None) -> None:
        """Attention over the pool; `window` is [B, Hkv, block] holding block pos // 64."""
        nb.sparse_decode_attn(self.dims, q, self.pool, self.pool_slots, self.phys, self.n_sel, self.k,
                              window, self.blk_elems, 0, pos, self.scale, self.out, self.ws_attn,
                              stream=stream)

    def attend_fetch(self, q: torch.Tensor, host_kv: torch.Tensor, window: torch.Tensor, pos: torch.Tensor,
                     insert_src: Optional[torch.Tensor] = None, stream=None) -> None:
        """nosa_sparse_decode_attn_fetch: the gather folded into the attention
        over the pool (after the step's pool update)."""
        nb.sparse_decode_attn_fetch(self.dims, q, host_kv, self.pool, self.pool_slots, self.phys, self.n_sel, self.k,
                                    self.miss_list, self.n_miss, insert_src, window, self.blk_elems, 0, pos,
                                    self.scale, self.out, self.ws_attn, stream=stream)

    def step_resident(self, q, kv, pos, stream=None) -> None:
        self.select(q, pos, stream)
        self.attend_resident(q, kv, pos, stream)

    def step_fused(self, q, kv, pos, stream=None) -> None:
        """Selection and attention of one step in one launch (resident cache)."""
        if self.ws_step is None:
            self.ws_step = torch.zeros(nb.workspace_size(self.dims, nb.OP_STEP, 1, self.kq, self.ke),
                                       dtype=torch.uint8, device=self.dev)
        nb.decode_step(self.dims, q, pos, self.k_comp, self.e_blk, self.kq, self.ke, kv, self.scale,
                       self.sel, self.n_sel, self.out, self.ws_step, stream=stream)

    def step_timeouts(self) -> int:
        """Waits of the one-launch step that hit their bound so far (0 when
        every hand-off completed), read through nosa_step_timeouts on the
        current stream (synchronises)."""
        if self.ws_step is None:
            return 0
        out = torch.zeros(1, dtype=torch.int32, device=self.dev)
        nb.step_timeouts(self.dims, self.kq, self.ke, self.ws_step, out)
        return int(out.item())

    def step_offload(self, q, host_kv, window, pos, step: int, insert_block=None, insert_src=None,
                     side: Optional[torch.cuda.Stream] = None, fused_fetch: bool = True) -> None:
        """One offload step.  fused_fetch (the default): selection and pool
        update in one launch, then the gather folded into the attention (two
        launches, one stream).  Else, without a side stream: select -> fetch
        -> attention on one stream; with one: selection and pool update in
        one launch, then the gather on the side stream while the attention
        over the blocks already resident (and the window) runs on the compute
        stream; then the attention over the fetched blocks merges both."""
        main = torch.cuda.current_stream()
        if fused_fetch:
            self.select_update(q, pos, step, insert_block, main)
            self.attend_fetch(q, host_kv, window, pos, insert_src, main)
            return
        if side is None:
            self.select(q, pos, main)
            self.fetch(host_kv, step, insert_block, insert_src, main)
            self.attend_pool(q, window, pos, main)
            return
        self.select_update(q, pos, step, insert_block, main)
        side.wait_stream(main)
        self.gather(host_kv, insert_src, side)
        self.attend_pool_part(q, window, pos, 0, main)
        main.wait_stream(side)
        self.attend_pool_part(q, window, pos, 1, main)

    def select_update(self, q: torch.Tensor, pos: torch.Tensor, step: int,
                      insert_block: Optional[torch.Tensor] = None, stream=None) -> None:
        """nosa_select_update_pool: the selection and the pool update in one launch."""
        nb.select_update_pool(self.dims, q, pos, self.k_comp, self.e_blk, self.kq, self.ke, self.sel, self.n_sel,
                              self.ws_sel, self.pool_slots, self.block_table, self.slot_block, self.slot_last_use,
                              step, insert_block, self.phys, self.miss_list, self.n_miss, stream=stream)

    def update_pool(self, step: int, insert_block: Optional[torch.Tensor] = None, stream=None) -> None:
        nb.update_pool(self.dims, self.pool_slots, self.block_table, self.slot_block, self.slot_last_use, step,
                       self.sel, self.n_sel, self.k, insert_block, self.phys, self.miss_list, self.n_miss,
                       stream=stream)

    def gather(self, host_kv: torch.Tensor, insert_src: Optional[torch.Tensor] = None, stream=None) -> None:
        nb.gather_blocks(self.dims, host_kv, self.pool, self.pool_slots, self.k, insert_src, self.miss_list,
                         self.n_miss, stream=stream)

    def attend_pool_part(self, q: torch.Tensor, window: torch.Tensor, pos: torch.Tensor, part: int,
                         stream=None) -> None:
        nb.sparse_decode_attn_pool(self.dims, q, self.pool, self.pool_slots, self.phys, self.n_sel, self.k,
                                   self.miss_list, self.n_miss, window, self.blk_elems, 0, pos, self.scale, part,
                                   self.out, self.ws_attn, stream=stream)


class PinnedHost:
    """Pinned host memory of an exact size (hipHostMalloc through the HIP
    runtime torch has loaded), viewed as a CPU tensor.  torch's own pinned
    allocator rounds every request up to a power of two, which turns a
    56 GiB multi-layer cache into 64 GiB.  Keep this object alive as long as
    the tensor is used."""

    def __init__(self, shape, dtype: torch.dtype):
        import ctypes
        self._hip = ctypes.CDLL("libamdhip64.so.7")      # the copy already in the process
        n = int(np.prod(shape))
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        ptr = ctypes.c_void_p()
        rc = self._hip.hipHostMalloc(ctypes.byref(ptr), ctypes.c_size_t(nbytes), ctypes.c_uint(0))
        if rc != 0 or not ptr.value:
            raise RuntimeError(f"hipHostMalloc of {nbytes} bytes failed (error {rc})")
        self._ptr = ptr
        raw = np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctypes.c_uint8)), shape=(nbytes,))
        self.tensor = torch.from_numpy(raw).view(dtype).view(*shape)

    def __del__(self):
        if getattr(self, "_ptr", None) is not None and self._ptr.value:
            self.tensor = None
            self._hip.hipHostFree(self._ptr)
            self._ptr = None


class OffloadStack:
    """Several attention layers decoding together in offload mode.

    Each layer keeps its KV cache in pinned host memory, its own HBM pool of
    `pool_slots` blocks per KV head and its own compressed keys; a decode
    step runs the layers one after another (select -> fetch -> attention per
    layer), the order a model's layers impose, since a layer's query exists
    only once the layer below has produced its output.
    """

    def __init__(self, n_layers: int, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 n_blocks: int, dtype: str, kq: int, ke: int, pool_slots: int, device: str = "cuda"):
        self.layers = [DecodeLayer(batch, n_q_heads, n_kv_heads, head_dim, n_blocks, dtype, kq, ke,
                                   pool_slots=pool_slots, device=device) for _ in range(n_layers)]
        L0 = self.layers[0]
        # one pinned allocation of the exact size for every layer
        self._pinned = PinnedHost((n_layers, batch, n_kv_heads, n_blocks, L0.blk_elems), L0.tdt)
        self.host_all = self._pinned.tensor
        self.host = [self.host_all[l] for l in range(n_layers)]     # pinned [B, Hkv, NB, block]
        self.logits = [None] * n_layers      # device [B, Hkv, NB * 64] fp32
        self.windows = [{} for _ in range(n_layers)]
        self.block = None                    # window block of the last step

    def load_layer(self, l: int, K: np.ndarray, V: np.ndarray, lam: np.ndarray, prompt_blocks,
                   window_blocks) -> None:
        """Layer l's cache from K, V [B, Hkv, T, D] and logits [B, Hkv, T]
        (float32 arrays holding cache-dtype values): the compressed keys of
        blocks [0, prompt_blocks) are pooled on the GPU, the listed window
        blocks stay in HBM, and the packed cache moves to pinned host memory.
        prompt_blocks is one count for the batch, or one per batch entry
        (entries at their own positions)."""
        L = self.layers[l]
        kv = to_device_blocks(K, V, L.NB, L.dtype, device=L.dev)
        logits = pad_logits(torch.from_numpy(lam).to(L.dev), L.NB)
        pb = np.broadcast_to(np.asarray(prompt_blocks, dtype=np.int64), (L.B,))
        lo, hi = int(pb.min()), int(pb.max())
        L.pool_blocks(kv, logits, 0, lo)
        for j in range(lo, hi):            # blocks complete for some entries only
            L.pool_entries(kv, logits, torch.from_numpy(np.where(j < pb, j, -1).astype(np.int32)).to(L.dev))
        self.windows[l] = {int(c): kv[:, :, int(c)].clone() for c in window_blocks}
        self.host[l].copy_(kv)
        self.logits[l] = logits
        self.block = (prompt_blocks if lo == hi and np.ndim(prompt_blocks) == 0 else pb.copy()) \
            if self.block is None else self.block
        del kv

    def _per_entry(self, l: int, blocks: np.ndarray) -> torch.Tensor:
        """[B, Hkv, block]: entry b's block blocks[b] of layer l's window buffers."""
        return torch.stack([self.windows[l][int(c)][b] for b, c in enumerate(blocks)])

    def step(self, t: int, qs, pos: torch.Tensor, block: int, side: Optional[torch.cuda.Stream] = None,
             on_layer=None, fetch_events=None, fused_update: bool = True, fused_fetch: bool = True) -> None:
        """Decode step t of every layer: qs[l] is layer l's query [B, Hq, D],
        pos [B] int32 the positions, inside window block `block` (one for the
        batch, or one per batch entry).  When an entry's window has moved on,
        the block it left is complete: its compressed keys are built and it
        enters that entry's pool.  on_layer(l, layer) runs after
        each layer is enqueued; fetch_events[l] (a list) gets the (start, end)
        event pair around that layer's gather (with no side stream, around
        its pool update and gather).  fused_update: the selection and the
        pool update as one launch (nosa_select_update_pool), else as two.
        fused_fetch: the gather folded into the attention
        (nosa_sparse_decode_attn_fetch) on the compute stream, after the
        one-launch selection and update; the side stream is not used and
        fetch_events[l] gets the pair around that attention."""
        ragged = np.ndim(block) > 0 or np.ndim(self.block) > 0
        B = self.layers[0].B
        cur = np.broadcast_to(np.asarray(block, dtype=np.int64), (B,)).copy()
        prev = np.broadcast_to(np.asarray(self.block, dtype=np.int64), (B,))
        if np.any(cur < prev) or np.any(cur > prev + 1):
            # one position per step: a window moves on by at most one block,
            # and the block it leaves is the only one to pool and insert
            raise ValueError(f"window blocks {cur.tolist()} after {prev.tolist()}: each must stay or move on by one")
        main = torch.cuda.current_stream()
        if ragged:
            moved = cur > prev
            entry_done = torch.from_numpy(np.where(moved, prev, -1).astype(np.int32)).to(self.layers[0].dev)
        else:
            done = self.block if block > self.block else None
        for l, L in enumerate(self.layers):
            ins_blk = ins_src = None
            if ragged:
                window = self._per_entry(l, cur)
                if moved.any():
                    ins_src = self._per_entry(l, np.where(moved, prev, cur))
                    L.pool_entries(ins_src, self.logits[l], entry_done, L.blk_elems, 0, main)
                    ins_blk = entry_done
            else:
                window = self.windows[l][block]
                if done is not None:
                    L.pool_window(self.windows[l][done], self.logits[l], done, main)
                    ins_blk = torch.full((L.B,), done, dtype=torch.int32, device=L.dev)
                    ins_src = self.windows[l][done]
            ev = None
            if fetch_events is not None:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            if fused_fetch:
                L.select_update(qs[l], pos, t, ins_blk, main)
                if ev is not None:
                    ev[0].record(main)
                L.attend_fetch(qs[l], self.host[l], window, pos, ins_src, main)
                if ev is not None:
                    ev[1].record(main)
            elif side is None:
                L.select(qs[l], pos, main)
                if ev is not None:
                    ev[0].record(main)
                L.fetch(self.host[l], t, ins_blk, ins_src, main)
                if ev is not None:
                    ev[1].record(main)
                L.attend_pool(qs[l], window, pos, main)
            else:
                # the gather on the side stream, the attention over the resident
                # blocks meanwhile (see DecodeLayer.step_offload)
                if fused_update:
                    L.select_update(qs[l], pos, t, ins_blk, main)
                else:
                    L.select(qs[l], pos, main)
                    L.update_pool(t, ins_blk, main)
                side.wait_stream(main)
                if ev is not None:
                    ev[0].record(side)
                L.gather(self.host[l], ins_src, side)
                if ev is not None:
                    ev[1].record(side)
                L.attend_pool_part(qs[l], window, pos, 0, main)
                main.wait_stream(side)
                L.attend_pool_part(qs[l], window, pos, 1, main)
            if ev is not None:
                fetch_events[l].append(ev)
            if on_layer is not None:
                on_layer(l, L)
        self.block = cur if ragged else block


def to_device_blocks(K: np.ndarray, V: np.ndarray, n_blocks: int, dtype: str, device="cuda") -> torch.Tensor:
    """numpy K, V [B, Hkv, T, D] (float32 holding cache-dtype values) -> packed device blocks."""
    tdt = torch_dtype(dtype)
    Kt = torch.from_numpy(K).to(device=device, dtype=tdt)
    Vt = torch.from_numpy(V).to(device=device, dtype=tdt)
    return pack_kv_blocks(Kt, Vt, n_blocks)
