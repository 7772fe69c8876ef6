"""ctypes binding of libnosa (the NOSA decode path on gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Buffers are torch tensors (device memory or pinned host memory) or
raw pointers; the stream defaults to torch's current stream.  A missing or
unloadable library raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnosa.so")

BLOCK = 64
SUB = 16
BF16, F32 = 0, 1
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, -1, -2, -3, -4
OP_SELECT, OP_ATTN, OP_STEP = 1, 2, 3

EXPORTS = ("nosa_pool_keys", "nosa_select_blocks", "nosa_fetch_blocks",
           "nosa_sparse_decode_attn", "nosa_decode_step", "nosa_workspace_size",
           "nosa_status_str", "nosa_last_error", "nosa_update_pool", "nosa_gather_blocks",
           "nosa_sparse_decode_attn_pool", "nosa_sparse_chunk_attn", "nosa_split_qkv",
           "nosa_select_blocks_shared", "nosa_step_timeouts", "nosa_decode_step_static",
           "nosa_select_blocks_fill", "nosa_sparse_decode_attn_bias", "nosa_pool_keys_entries",
           "nosa_select_update_pool", "nosa_sparse_decode_attn_fetch", "nosa_debug_expire_step_waits")


class NosaError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} returned {code}: {text}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnosa.so once (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run kv_cache_offload_amd.build.build() first")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(Dims)
    lib.nosa_pool_keys.argtypes = [D, P, I64, I64, P, I32, I32, P, P, P, P]
    lib.nosa_pool_keys_entries.argtypes = [D, P, I64, I64, P, P, P, P, P, P]
    lib.nosa_select_blocks.argtypes = [D, P, I32, P, P, P, I32, I32, P, P, P, SZ, P]
    lib.nosa_select_blocks_shared.argtypes = [D, P, I32, P, P, P, I32, I32, P, P, P, SZ, P]
    lib.nosa_select_blocks_fill.argtypes = [D, P, I32, P, P, P, I32, I32, P, P, P, SZ, P]
    lib.nosa_sparse_decode_attn_bias.argtypes = [D, P, P, P, P, I32, P, F, P, P, P, SZ, P]
    lib.nosa_fetch_blocks.argtypes = [D, P, P, I32, P, P, P, I32, P, P, I32, P, P, P, P, P, P]
    lib.nosa_sparse_decode_attn.argtypes = [D, P, P, I32, P, P, I32, P, I64, I64, P, F, P, P, SZ, P]
    lib.nosa_decode_step.argtypes = [D, P, P, P, P, I32, I32, P, F, P, P, P, P, SZ, P]
    lib.nosa_workspace_size.argtypes = [D, I32, I32, I32, I32]
    lib.nosa_update_pool.argtypes = [D, I32, P, P, P, I32, P, P, I32, P, P, P, P, P]
    lib.nosa_sparse_decode_attn_fetch.argtypes = [D, P, P, P, I32, P, P, I32, P, P, P, P, I64, I64, P, F, P, P, SZ, P]
    lib.nosa_select_update_pool.argtypes = [D, P, P, P, P, I32, I32, P, P, P, SZ, I32, P, P, P, I32, P, P, P, P, P]
    lib.nosa_gather_blocks.argtypes = [D, P, P, I32, I32, P, P, P, P]
    lib.nosa_sparse_decode_attn_pool.argtypes = [D, P, P, I32, P, P, I32, P, P, P, I64, I64, P, F, I32, P, P, SZ, P]
    lib.nosa_sparse_chunk_attn.argtypes = [D, P, I32, P, P, P, I32, P, F, P, P, SZ, P]
    lib.nosa_split_qkv.argtypes = [D, P, I32, P, P, P, I32, P, P, P, P]
    lib.nosa_step_timeouts.argtypes = [D, I32, I32, P, P, P]
    lib.nosa_decode_step_static.argtypes = [D, P, P, P, P, I32, I32, P, F, P, P, P, P]
    lib.nosa_debug_expire_step_waits.argtypes = [I32]
    lib.nosa_workspace_size.restype = SZ
    lib.nosa_status_str.argtypes = [I32]
    lib.nosa_status_str.restype = ctypes.c_char_p
    lib.nosa_last_error.argtypes = []
    lib.nosa_last_error.restype = ctypes.c_char_p
    for name in ("nosa_pool_keys", "nosa_select_blocks", "nosa_fetch_blocks", "nosa_sparse_decode_attn",
                 "nosa_decode_step", "nosa_update_pool", "nosa_gather_blocks", "nosa_sparse_decode_attn_pool",
                 "nosa_sparse_chunk_attn", "nosa_split_qkv", "nosa_select_blocks_shared", "nosa_step_timeouts", "nosa_decode_step_static",
                 "nosa_select_blocks_fill", "nosa_sparse_decode_attn_bias", "nosa_pool_keys_entries",
           "nosa_select_update_pool", "nosa_sparse_decode_attn_fetch", "nosa_debug_expire_step_waits"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def dims(batch, n_q_heads, n_kv_heads, head_dim, max_blocks, dtype) -> Dims:
    code = {"bf16": BF16, "f32": F32}.get(dtype, dtype)
    return Dims(batch, n_q_heads, n_kv_heads, head_dim, max_blocks, code)


def _ptr(x) -> Optional[int]:
    """Address of a tensor's data, an int address, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != OK:
        lib = load()
        raise NosaError(fn, rc, lib.nosa_last_error().decode())


def workspace_size(d: Dims, op: int, n_query: int, kq: int, ke: int) -> int:
    return int(load().nosa_workspace_size(ctypes.byref(d), op, n_query, kq, ke))


def split_qkv(d: Dims, qkv, n_tok: int, pos, w1, w2, d_e: int, q_out, kv, evict_logits, stream=None) -> None:
    rc = load().nosa_split_qkv(ctypes.byref(d), _ptr(qkv), n_tok, _ptr(pos), _ptr(w1), _ptr(w2), d_e, _ptr(q_out),
                               _ptr(kv), _ptr(evict_logits), _stream(stream))
    _check("nosa_split_qkv", rc)


def pool_keys(d: Dims, kv, kv_unit_stride: int, kv_block_stride: int, evict_logits,
              blk_begin: int, blk_end: int, k_comp, e_sub, e_blk, stream=None) -> None:
    rc = load().nosa_pool_keys(ctypes.byref(d), _ptr(kv), kv_unit_stride, kv_block_stride,
                               _ptr(evict_logits), blk_begin, blk_end, _ptr(k_comp), _ptr(e_sub),
                               _ptr(e_blk), _stream(stream))
    _check("nosa_pool_keys", rc)


def pool_keys_entries(d: Dims, kv, kv_unit_stride: int, kv_block_stride: int, evict_logits, entry_block,
                      k_comp, e_sub, e_blk, stream=None) -> None:
    rc = load().nosa_pool_keys_entries(ctypes.byref(d), _ptr(kv), kv_unit_stride, kv_block_stride,
                                       _ptr(evict_logits), _ptr(entry_block), _ptr(k_comp), _ptr(e_sub),
                                       _ptr(e_blk), _stream(stream))
    _check("nosa_pool_keys_entries", rc)


def select_blocks(d: Dims, q, n_query: int, pos, k_comp, e_blk, kq: int, ke: int, sel, n_sel,
                  ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_select_blocks(ctypes.byref(d), _ptr(q), n_query, _ptr(pos), _ptr(k_comp),
                                   _ptr(e_blk), kq, ke, _ptr(sel), _ptr(n_sel), _ptr(ws), ws_bytes,
                                   _stream(stream))
    _check("nosa_select_blocks", rc)


def select_blocks_fill(d: Dims, q, n_query: int, pos, k_comp, e_blk, kq: int, ke: int, sel, n_sel,
                       ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_select_blocks_fill(ctypes.byref(d), _ptr(q), n_query, _ptr(pos), _ptr(k_comp),
                                        _ptr(e_blk), kq, ke, _ptr(sel), _ptr(n_sel), _ptr(ws), ws_bytes,
                                        _stream(stream))
    _check("nosa_select_blocks_fill", rc)


def sparse_decode_attn_bias(d: Dims, q, kv, sel, n_sel, k_cap: int, pos, scale: Optional[float], evict_logits,
                            out, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if scale is None:
        scale = 1.0 / math.sqrt(d.head_dim)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_sparse_decode_attn_bias(ctypes.byref(d), _ptr(q), _ptr(kv), _ptr(sel), _ptr(n_sel), k_cap,
                                             _ptr(pos), float(scale), _ptr(evict_logits), _ptr(out), _ptr(ws),
                                             ws_bytes, _stream(stream))
    _check("nosa_sparse_decode_attn_bias", rc)


def select_blocks_shared(d: Dims, q, n_query: int, pos, k_comp, e_blk, kq: int, ke: int, sel, n_sel,
                         ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_select_blocks_shared(ctypes.byref(d), _ptr(q), n_query, _ptr(pos), _ptr(k_comp),
                                          _ptr(e_blk), kq, ke, _ptr(sel), _ptr(n_sel), _ptr(ws), ws_bytes,
                                          _stream(stream))
    _check("nosa_select_blocks_shared", rc)


def fetch_blocks(d: Dims, host_kv, pool, pool_slots: int, block_table, slot_block, slot_last_use,
                 step: int, sel, n_sel, k_cap: int, insert_block, insert_src, phys, miss_list,
                 n_miss, stream=None) -> None:
    rc = load().nosa_fetch_blocks(ctypes.byref(d), _ptr(host_kv), _ptr(pool), pool_slots,
                                  _ptr(block_table), _ptr(slot_block), _ptr(slot_last_use), step,
                                  _ptr(sel), _ptr(n_sel), k_cap, _ptr(insert_block),
                                  _ptr(insert_src), _ptr(phys), _ptr(miss_list), _ptr(n_miss),
                                  _stream(stream))
    _check("nosa_fetch_blocks", rc)


def update_pool(d: Dims, pool_slots: int, block_table, slot_block, slot_last_use, step: int, sel, n_sel,
                k_cap: int, insert_block, phys, miss_list, n_miss, stream=None) -> None:
    rc = load().nosa_update_pool(ctypes.byref(d), pool_slots, _ptr(block_table), _ptr(slot_block),
                                 _ptr(slot_last_use), step, _ptr(sel), _ptr(n_sel), k_cap, _ptr(insert_block),
                                 _ptr(phys), _ptr(miss_list), _ptr(n_miss), _stream(stream))
    _check("nosa_update_pool", rc)


def select_update_pool(d: Dims, q, pos, k_comp, e_blk, kq: int, ke: int, sel, n_sel, ws, pool_slots: int,
                       block_table, slot_block, slot_last_use, step: int, insert_block, phys, miss_list, n_miss,
                       ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_select_update_pool(ctypes.byref(d), _ptr(q), _ptr(pos), _ptr(k_comp), _ptr(e_blk), kq, ke,
                                        _ptr(sel), _ptr(n_sel), _ptr(ws), ws_bytes, pool_slots, _ptr(block_table),
                                        _ptr(slot_block), _ptr(slot_last_use), step, _ptr(insert_block),
                                        _ptr(phys), _ptr(miss_list), _ptr(n_miss), _stream(stream))
    _check("nosa_select_update_pool", rc)


def gather_blocks(d: Dims, host_kv, pool, pool_slots: int, k_cap: int, insert_src, miss_list, n_miss,
                  stream=None) -> None:
    rc = load().nosa_gather_blocks(ctypes.byref(d), _ptr(host_kv), _ptr(pool), pool_slots, k_cap,
                                   _ptr(insert_src), _ptr(miss_list), _ptr(n_miss), _stream(stream))
    _check("nosa_gather_blocks", rc)


def sparse_decode_attn_fetch(d: Dims, q, host_kv, pool, pool_slots: int, phys, n_sel, k_cap: int, miss_list, n_miss,
                             insert_src, window_kv, window_head_stride: int, window_block_stride: int, pos,
                             scale: Optional[float], out, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if scale is None:
        scale = 1.0 / math.sqrt(d.head_dim)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_sparse_decode_attn_fetch(ctypes.byref(d), _ptr(q), _ptr(host_kv), _ptr(pool), pool_slots,
                                              _ptr(phys), _ptr(n_sel), k_cap, _ptr(miss_list), _ptr(n_miss),
                                              _ptr(insert_src), _ptr(window_kv), window_head_stride,
                                              window_block_stride, _ptr(pos), scale, _ptr(out), _ptr(ws), ws_bytes,
                                              _stream(stream))
    _check("nosa_sparse_decode_attn_fetch", rc)


def sparse_decode_attn_pool(d: Dims, q, pool, pool_slots: int, phys, n_sel, k_cap: int, miss_list, n_miss,
                            window_kv, window_head_stride: int, window_block_stride: int, pos,
                            scale: Optional[float], part: int, out, ws, ws_bytes: Optional[int] = None,
                            stream=None) -> None:
    if scale is None:
        scale = 1.0 / math.sqrt(d.head_dim)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_sparse_decode_attn_pool(ctypes.byref(d), _ptr(q), _ptr(pool), pool_slots, _ptr(phys),
                                             _ptr(n_sel), k_cap, _ptr(miss_list), _ptr(n_miss), _ptr(window_kv),
                                             window_head_stride, window_block_stride, _ptr(pos), scale, part,
                                             _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    _check("nosa_sparse_decode_attn_pool", rc)


def sparse_chunk_attn(d: Dims, q, n_query: int, kv, sel, n_sel, k_cap: int, pos, scale: Optional[float], out, ws,
                      ws_bytes: Optional[int] = None, stream=None) -> None:
    if scale is None:
        scale = 1.0 / math.sqrt(d.head_dim)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_sparse_chunk_attn(ctypes.byref(d), _ptr(q), n_query, _ptr(kv), _ptr(sel), _ptr(n_sel), k_cap,
                                       _ptr(pos), scale, _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    _check("nosa_sparse_chunk_attn", rc)


def sparse_decode_attn(d: Dims, q, blocks, blocks_per_head: int, phys, n_sel, k_cap: int,
                       window_kv, window_head_stride: int, window_block_stride: int, pos,
                       scale: Optional[float], out, ws, ws_bytes: Optional[int] = None,
                       stream=None) -> None:
    if scale is None:
        scale = 1.0 / math.sqrt(d.head_dim)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_sparse_decode_attn(ctypes.byref(d), _ptr(q), _ptr(blocks), blocks_per_head,
                                        _ptr(phys), _ptr(n_sel), k_cap, _ptr(window_kv),
                                        window_head_stride, window_block_stride, _ptr(pos),
                                        float(scale), _ptr(out), _ptr(ws), ws_bytes,
                                        _stream(stream))
    _check("nosa_sparse_decode_attn", rc)


def decode_step(d: Dims, q, pos, k_comp, e_blk, kq: int, ke: int, kv, scale: Optional[float], sel,
                n_sel, out, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if scale is None:
        scale = 1.0 / math.sqrt(d.head_dim)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    rc = load().nosa_decode_step(ctypes.byref(d), _ptr(q), _ptr(pos), _ptr(k_comp), _ptr(e_blk), kq, ke,
                                 _ptr(kv), float(scale), _ptr(sel), _ptr(n_sel), _ptr(out), _ptr(ws),
                                 ws_bytes, _stream(stream))
    _check("nosa_decode_step", rc)


def step_timeouts(d: Dims, kq: int, ke: int, ws, out, stream=None) -> None:
    """Enqueue the copy of workspace ws's hand-off timeout count into out
    (an int32 device or pinned host tensor)."""
    rc = load().nosa_step_timeouts(ctypes.byref(d), kq, ke, _ptr(ws), _ptr(out), _stream(stream))
    _check("nosa_step_timeouts", rc)


def debug_expire_step_waits(on: bool) -> None:
    """Test hook: while on, the one-launch step's score waits expire (counted, NaN outputs)."""
    _check("nosa_debug_expire_step_waits", load().nosa_debug_expire_step_waits(1 if on else 0))


def decode_step_static(d: Dims, q, pos, k_comp, e_blk, kq: int, ke: int, kv, scale: Optional[float], sel, n_sel,
                       out, stream=None) -> None:
    """nosa_decode_step on the library's own per-device workspace (no allocation)."""
    if scale is None:
        scale = 1.0 / math.sqrt(d.head_dim)
    rc = load().nosa_decode_step_static(ctypes.byref(d), _ptr(q), _ptr(pos), _ptr(k_comp), _ptr(e_blk), kq, ke,
                                        _ptr(kv), float(scale), _ptr(sel), _ptr(n_sel), _ptr(out), _stream(stream))
    _check("nosa_decode_step_static", rc)
