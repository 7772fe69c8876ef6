"""Decode-step driver: device buffers of one attention layer and the order of
the four libnosa calls per step.

Two modes:

* resident -- the whole KV cache of the layer sits in HBM; attention reads
  the selected blocks in place (phys = the selected block ids) and the
  window straight from the cache;
* offload  -- the KV cache sits in pinned host memory; a fixed HBM pool of
  `pool_slots` blocks per KV head holds the selected blocks, refilled each
  step by nosa_fetch_blocks on a side stream (NOSI's design: only the window
  and the Top-K blocks stay on the GPU, the rest is offloaded).

Per step: select (compute stream) -> [fetch (side stream)] -> attention
(compute stream).  The compressed keys of a block are built once, when the
block is complete.  All buffers are torch tensors; torch provides device
memory, pinned host memory and streams, and nothing else.
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

    # -- one decode step -------------------------------------------------
    def select(self, q: torch.Tensor, pos: torch.Tensor, stream=None) -> None:
        nb.select_blocks(self.dims, q, 1, pos, self.k_comp, self.e_blk, self.kq, self.ke, self.sel,
                         self.n_sel, self.ws_sel, stream=stream)

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
        every hand-off completed); reads the workspace counter (synchronises)."""
        if self.ws_step is None:
            return 0
        units = self.dims.batch * self.dims.n_kv_heads
        off = (units * 4 + 255) // 256 * 256
        return int(self.ws_step[off:off + 4].view(torch.int32).item())

    def step_offload(self, q, host_kv, window, pos, step: int, insert_block=None, insert_src=None,
                     side: Optional[torch.cuda.Stream] = None) -> None:
        """select -> fetch on the side stream -> attention, ordered with events."""
        main = torch.cuda.current_stream()
        self.select(q, pos, main)
        if side is None:
            self.fetch(host_kv, step, insert_block, insert_src, main)
        else:
            side.wait_stream(main)
            self.fetch(host_kv, step, insert_block, insert_src, side)
            main.wait_stream(side)
        self.attend_pool(q, window, pos, main)


def to_device_blocks(K: np.ndarray, V: np.ndarray, n_blocks: int, dtype: str, device="cuda") -> torch.Tensor:
    """numpy K, V [B, Hkv, T, D] (float32 holding cache-dtype values) -> packed device blocks."""
    tdt = torch_dtype(dtype)
    Kt = torch.from_numpy(K).to(device=device, dtype=tdt)
    Vt = torch.from_numpy(V).to(device=device, dtype=tdt)
    return pack_kv_blocks(Kt, Vt, n_blocks)
