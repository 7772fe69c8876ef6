"""The C ABI without a GPU: the library loads, exports what nosa.h declares,
and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

from kv_cache_offload_amd import binding as nb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nb.LIB_PATH):
        from kv_cache_offload_amd import build
        build.build()
    return nb.load()


def _declared():
    text = open(os.path.join(ROOT, "include", "nosa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(nosa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    names = _declared()
    for fn in ("nosa_pool_keys", "nosa_select_blocks", "nosa_fetch_blocks", "nosa_sparse_decode_attn",
               "nosa_decode_step"):
        assert fn in names
    assert sorted(nb.EXPORTS) == names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.nosa_status_str(0) == b"ok"
    assert lib.nosa_status_str(-4) == b"workspace too small"
    assert lib.nosa_status_str(12345) == b"unknown status"


def _d(**kw):
    base = dict(batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128, max_blocks=64, dtype="bf16")
    base.update(kw)
    return nb.dims(**base)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_workspace_sizes(lib):
    d = _d()
    s = nb.workspace_size(d, nb.OP_SELECT, 1, 16, 48)
    a = nb.workspace_size(d, nb.OP_ATTN, 1, 16, 48)
    assert s >= 2 * 2 * 64 * 4 and a > 0          # one fp32 score per block and row
    assert nb.workspace_size(d, 99, 1, 16, 48) == 0
    assert nb.workspace_size(_d(head_dim=96), nb.OP_ATTN, 1, 16, 48) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=96), nb.ERR_UNSUPPORTED),
    (dict(dtype=7), nb.ERR_UNSUPPORTED),
    (dict(n_q_heads=15), nb.ERR_ARG),
    (dict(n_q_heads=64, n_kv_heads=2), nb.ERR_UNSUPPORTED),
    (dict(batch=0), nb.ERR_ARG),
    (dict(max_blocks=0), nb.ERR_ARG),
])
def test_bad_dims_rejected(lib, bad, code):
    d = _d(**bad)
    with pytest.raises(nb.NosaError) as e:
        nb.pool_keys(d, FAKE, 0, 0, FAKE, 0, 1, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == code


def test_pool_keys_range_checked(lib):
    for lo, hi in ((-1, 2), (3, 2), (0, 65)):
        with pytest.raises(nb.NosaError) as e:
            nb.pool_keys(_d(), FAKE, 0, 0, FAKE, lo, hi, FAKE, FAKE, FAKE, stream=0)
        assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.pool_keys(_d(), None, 0, 0, FAKE, 0, 1, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG and "NULL" in str(e.value)
    with pytest.raises(nb.NosaError) as e:
        nb.pool_keys(_d(), FAKE, -1, 0, FAKE, 0, 1, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG


def test_select_checks(lib):
    d = _d()
    need = nb.workspace_size(d, nb.OP_SELECT, 1, 4, 4)
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks(d, FAKE, 1, FAKE, FAKE, FAKE, 4, 4, FAKE, FAKE, FAKE, need - 1, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks(d, FAKE, 1, FAKE, FAKE, FAKE, -1, 4, FAKE, FAKE, FAKE, need, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks(d, FAKE, 0, FAKE, FAKE, FAKE, 4, 4, FAKE, FAKE, FAKE, need, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks(_d(max_blocks=5000), FAKE, 1, FAKE, FAKE, FAKE, 4, 4, FAKE, FAKE, FAKE,
                         1 << 40, stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED


def test_select_shared_checks(lib):
    """The chunk-shared selection validates like nosa_select_blocks, and
    rejects fp32 caches and query groups other than 1, 2, 4 or 8 heads."""
    d = _d()
    need = nb.workspace_size(d, nb.OP_SELECT, 1, 4, 4)
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks_shared(d, FAKE, 1, FAKE, FAKE, FAKE, 4, 4, FAKE, FAKE, FAKE, need - 1, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks_shared(d, FAKE, 0, FAKE, FAKE, FAKE, 4, 4, FAKE, FAKE, FAKE, need, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks_shared(_d(dtype=nb.F32), FAKE, 8, FAKE, FAKE, FAKE, 4, 4, FAKE, FAKE, FAKE, 1 << 40,
                                stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks_shared(_d(n_q_heads=24, n_kv_heads=2), FAKE, 8, FAKE, FAKE, FAKE, 4, 4, FAKE, FAKE,
                                FAKE, 1 << 40, stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED


def test_select_workspace_covers_shared_selection(lib):
    """The selection workspace also holds what the chunk-shared selection
    keeps there: one score per (unit, block) and 16 partial query sums of up
    to 128 fp32 dimensions per unit, after the per-row tickets."""
    for n_query in (1, 2, 9, 64):
        d = _d(max_blocks=2048)
        need = nb.workspace_size(d, nb.OP_SELECT, n_query, 16, 48)
        units = d.batch * d.n_kv_heads
        assert need >= units * n_query * 4 + units * 2048 * 4 + 16 * units * 128 * 4


def test_fetch_checks(lib):
    d = _d()
    args = lambda P, k: (d, FAKE, FAKE, P, FAKE, FAKE, FAKE, 0, FAKE, FAKE, k, None, None, FAKE, FAKE, FAKE)
    with pytest.raises(nb.NosaError) as e:
        nb.fetch_blocks(*args(64, 64), stream=0)          # pool must exceed k
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.fetch_blocks(*args(80, 65), stream=0)          # one wavefront holds S
    assert e.value.code == nb.ERR_UNSUPPORTED
    with pytest.raises(nb.NosaError) as e:
        nb.fetch_blocks(*args(2000, 8), stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED
    a = list(args(80, 64))
    a[11] = FAKE                                          # insert_block without insert_src
    with pytest.raises(nb.NosaError) as e:
        nb.fetch_blocks(*a, stream=0)
    assert e.value.code == nb.ERR_ARG


def test_attn_checks(lib):
    d = _d()
    need = nb.workspace_size(d, nb.OP_ATTN, 1, 64, 0)
    base = [d, FAKE, FAKE, 64, FAKE, FAKE, 64, FAKE, 64 * 32768, 32768, FAKE, None, FAKE, FAKE]
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_decode_attn(*base, ws_bytes=need - 1, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE
    bad = list(base)
    bad[8] = -1
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_decode_attn(*bad, ws_bytes=need, stream=0)
    assert e.value.code == nb.ERR_ARG
    bad = list(base)
    bad[11] = float("nan")
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_decode_attn(*bad, ws_bytes=need, stream=0)
    assert e.value.code == nb.ERR_ARG
    assert "scale" in lib.nosa_last_error().decode()


def test_split_fetch_and_pool_attention_checks(lib):
    d = _d()
    with pytest.raises(nb.NosaError) as e:                # pool must exceed k
        nb.update_pool(d, 64, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 64, None, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:                # the tables are required
        nb.update_pool(d, 80, None, FAKE, FAKE, 0, FAKE, FAKE, 64, None, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:                # the host cache is required
        nb.gather_blocks(d, None, FAKE, 80, 64, None, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.gather_blocks(d, FAKE, FAKE, 2000, 8, None, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED
    need = nb.workspace_size(d, nb.OP_ATTN, 1, 64, 0)
    base = [d, FAKE, FAKE, 80, FAKE, FAKE, 64, FAKE, FAKE, FAKE, 32768, 0, FAKE, None]
    for part in (-1, 2):
        with pytest.raises(nb.NosaError) as e:
            nb.sparse_decode_attn_pool(*base, part, FAKE, FAKE, ws_bytes=need, stream=0)
        assert e.value.code == nb.ERR_ARG
    bad = list(base)
    bad[7] = None                                         # the miss list is required
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_decode_attn_pool(*bad, 0, FAKE, FAKE, ws_bytes=need, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_decode_attn_pool(*base, 1, FAKE, FAKE, ws_bytes=need - 1, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE


def test_chunk_attn_checks(lib):
    d = _d()
    need = nb.workspace_size(d, nb.OP_ATTN, 8, 64, 0)
    assert need > nb.workspace_size(d, nb.OP_ATTN, 1, 64, 0)
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_chunk_attn(d, FAKE, 0, FAKE, FAKE, FAKE, 64, FAKE, None, FAKE, FAKE, ws_bytes=need, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_chunk_attn(d, FAKE, 8, FAKE, FAKE, FAKE, 64, FAKE, None, FAKE, FAKE, ws_bytes=need - 1, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_chunk_attn(_d(batch=64), FAKE, 1024, FAKE, FAKE, FAKE, 64, FAKE, None, FAKE, FAKE,
                             ws_bytes=1 << 40, stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED


def test_split_qkv_checks(lib):
    d = _d()
    args = lambda n_tok, d_e: (d, FAKE, n_tok, FAKE, FAKE, FAKE, d_e, FAKE, FAKE, FAKE)
    for n_tok, d_e, code in ((0, 64, nb.ERR_ARG), (8, 0, nb.ERR_UNSUPPORTED), (8, 513, nb.ERR_UNSUPPORTED)):
        with pytest.raises(nb.NosaError) as e:
            nb.split_qkv(*args(n_tok, d_e), stream=0)
        assert e.value.code == code
    a = list(args(8, 64))
    a[4] = None                                           # W1 is required
    with pytest.raises(nb.NosaError) as e:
        nb.split_qkv(*a, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.split_qkv(_d(n_q_heads=32, n_kv_heads=32), *args(8, 64)[1:], stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED


def test_step_checks(lib):
    d = _d()
    need = nb.workspace_size(d, nb.OP_STEP, 1, 16, 48)
    assert need > 0
    args = [d, FAKE, FAKE, FAKE, FAKE, 16, 48, FAKE, None, FAKE, FAKE, FAKE, FAKE]
    with pytest.raises(nb.NosaError) as e:
        nb.decode_step(*args, ws_bytes=need - 1, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE
    bad = list(args)
    bad[5], bad[6] = 200, 100
    with pytest.raises(nb.NosaError) as e:
        nb.decode_step(*bad, ws_bytes=1 << 30, stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED
    with pytest.raises(nb.NosaError) as e:
        nb.decode_step(_d(n_q_heads=32), *args[1:], ws_bytes=1 << 30, stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED


def test_step_timeouts_checks(lib):
    d = _d()
    for ws, out in ((None, FAKE), (FAKE, None)):
        with pytest.raises(nb.NosaError) as e:
            nb.step_timeouts(d, 16, 48, ws, out, stream=0)
        assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.step_timeouts(d, -1, 48, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG


def test_expire_hook_toggles_and_step_checks_still_apply(lib):
    # the failure-handling test hook only flips a flag; the step's argument
    # checks run as before while it is on, and it is off again afterwards
    assert lib.nosa_debug_expire_step_waits(1) == nb.OK
    try:
        with pytest.raises(nb.NosaError) as e:
            nb.decode_step(_d(), FAKE, FAKE, FAKE, FAKE, -1, 48, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                           stream=0)
        assert e.value.code == nb.ERR_ARG
    finally:
        assert lib.nosa_debug_expire_step_waits(0) == nb.OK


def test_static_step_rejects_a_workspace_above_its_size(lib):
    # 2048 units x 4096 blocks of scores alone need 64 MiB: more than the
    # static workspace holds; rejected before anything touches a device
    d = _d(batch=1024, max_blocks=4096)
    assert nb.workspace_size(d, nb.OP_STEP, 1, 16, 48) > (16 << 20)
    with pytest.raises(nb.NosaError) as e:
        nb.decode_step_static(d, FAKE, FAKE, FAKE, FAKE, 16, 48, FAKE, None, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE
    assert "16 MiB" in lib.nosa_last_error().decode()


def test_variant_calls_check_like_their_bases(lib):
    d = _d()
    need = nb.workspace_size(d, nb.OP_SELECT, 1, 16, 48)
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks_fill(d, FAKE, 1, FAKE, FAKE, FAKE, 16, 48, FAKE, FAKE, FAKE, ws_bytes=need - 1, stream=0)
    assert e.value.code == nb.ERR_WORKSPACE
    with pytest.raises(nb.NosaError) as e:
        nb.select_blocks_fill(d, FAKE, 0, FAKE, FAKE, FAKE, 16, 48, FAKE, FAKE, FAKE, ws_bytes=need, stream=0)
    assert e.value.code == nb.ERR_ARG
    need_a = nb.workspace_size(d, nb.OP_ATTN, 1, 64, 0)
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_decode_attn_bias(d, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, None, FAKE, FAKE, ws_bytes=need_a,
                                   stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.sparse_decode_attn_bias(d, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, FAKE, FAKE, FAKE, ws_bytes=need_a - 1,
                                   stream=0)
    assert e.value.code == nb.ERR_WORKSPACE


def test_pool_keys_entries_checks(lib):
    with pytest.raises(nb.NosaError) as e:
        nb.pool_keys_entries(_d(), FAKE, 0, 0, FAKE, None, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG and "entry_block" in str(e.value)
    with pytest.raises(nb.NosaError) as e:
        nb.pool_keys_entries(_d(), FAKE, -1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_ARG
    with pytest.raises(nb.NosaError) as e:
        nb.pool_keys_entries(_d(head_dim=96), FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == nb.ERR_UNSUPPORTED


def test_select_update_pool_checks(lib):
    """Both calls' checks, before anything is launched: the pool's k <= 64
    and pool_slots > k, the tables, and the selection's workspace."""
    d = _d()
    need = nb.workspace_size(d, nb.OP_SELECT, 1, 16, 48)

    def call(kq=16, ke=48, ws_bytes=need, P=80, bt=FAKE):
        nb.select_update_pool(d, FAKE, FAKE, FAKE, FAKE, kq, ke, FAKE, FAKE, FAKE, P, bt, FAKE, FAKE, 0, None,
                              FAKE, FAKE, FAKE, ws_bytes=ws_bytes, stream=0)

    for kw, code in ((dict(kq=16, ke=49), nb.ERR_UNSUPPORTED), (dict(kq=-1), nb.ERR_ARG),
                     (dict(P=64), nb.ERR_ARG), (dict(P=2000), nb.ERR_UNSUPPORTED), (dict(bt=None), nb.ERR_ARG),
                     (dict(ws_bytes=need - 1), nb.ERR_WORKSPACE)):
        with pytest.raises(nb.NosaError) as e:
            call(**kw)
        assert e.value.code == code, kw


def test_attention_fetch_checks(lib):
    d = _d()
    need = nb.workspace_size(d, nb.OP_ATTN, 1, 64, 0)

    def call(host=FAKE, k_cap=64, P=80, part_ws=need):
        nb.sparse_decode_attn_fetch(d, FAKE, host, FAKE, P, FAKE, FAKE, k_cap, FAKE, FAKE, None, FAKE, 0, 0, FAKE,
                                    None, FAKE, FAKE, ws_bytes=part_ws, stream=0)

    for kw, code in ((dict(host=None), nb.ERR_ARG), (dict(k_cap=65), nb.ERR_UNSUPPORTED), (dict(P=0), nb.ERR_ARG),
                     (dict(part_ws=need - 1), nb.ERR_WORKSPACE)):
        with pytest.raises(nb.NosaError) as e:
            call(**kw)
        assert e.value.code == code, kw
