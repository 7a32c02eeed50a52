"""Host-side checks of libinfllm.so, no GPU needed: the library loads, exports
every function include/infllm.h declares, and its validation returns the
documented status codes before any device work (fake, never-dereferenced
pointers are passed on purpose)."""
import ctypes
import os
import re

import pytest

from block_level_kv_amd import infllm as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infllm.h")

FAKE = 1 << 32          # 16-byte aligned, never dereferenced by validation
MISALIGNED = FAKE + 4


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"INFLLM_API\s+[^;(]*?\b(infllm_\w+)\s*\(", text)))


def cfg(**kw):
    base = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, block=128, n_init=128, window=4096,
                rep_k=4, top_k=16, rep_mode=F.INFLLM_REP_TOKENS, dtype=F.INFLLM_BF16)
    base.update(kw)
    return F.make_config(**base)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 16
    assert set(names) == set(F.EXPORTED)
    L = F.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.infllm_abi_version() == 1


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert F.status_string(code) and F.status_string(code) != "unknown status"
    assert F.status_string(7) == "unknown status"


def test_num_units_and_eligible_closed_forms():
    c = cfg()
    assert F.infllm_num_units(c, 131072) == 1023
    assert F.infllm_num_units(c, 1 << 20) == 8191
    assert F.infllm_num_units(c, 100) == 0
    c1 = cfg(n_q_heads=1, n_kv_heads=1, head_dim=64, n_init=64, window=512, top_k=4,
             dtype=F.INFLLM_F32)
    assert F.infllm_num_units(c1, 4096) == 32
    # first key of unit 0 is n_init; of unit u >= 1 it is (u + n_init//B) * B
    for t_last in (0, 4223, 4224, 4351, 4352, 50000, 200000):
        x = t_last - 4096
        want = 0 if x < 128 else min(1023, x // 128)
        assert F.infllm_num_eligible(c, t_last, 1023) == want
    for t_last in range(0, 4096, 17):
        x = t_last - 512
        want = 0 if x < 64 else min(32, x // 128 + 1)
        assert F.infllm_num_eligible(c1, t_last, 32) == want
    assert F.infllm_num_units(cfg(n_kv_heads=5), 100) == -1


@pytest.mark.parametrize("field,value,code", [
    ("n_kv_heads", 0, F.INFLLM_ERR_INVALID_ARG),
    ("n_kv_heads", 3, F.INFLLM_ERR_INVALID_ARG),       # 32 % 3 != 0
    ("n_q_heads", 48, F.INFLLM_ERR_UNSUPPORTED),      # G = 6
    ("head_dim", 96, F.INFLLM_ERR_UNSUPPORTED),
    ("head_dim", 0, F.INFLLM_ERR_INVALID_ARG),
    ("block", 100, F.INFLLM_ERR_UNSUPPORTED),
    ("window", 0, F.INFLLM_ERR_INVALID_ARG),
    ("n_init", -1, F.INFLLM_ERR_INVALID_ARG),
    ("rep_k", 0, F.INFLLM_ERR_INVALID_ARG),
    ("rep_k", 129, F.INFLLM_ERR_INVALID_ARG),
    ("top_k", -1, F.INFLLM_ERR_INVALID_ARG),
    ("top_k", 300, F.INFLLM_ERR_UNSUPPORTED),
    ("dtype", 5, F.INFLLM_ERR_INVALID_ARG),
    ("rep_mode", 2, F.INFLLM_ERR_INVALID_ARG),
])
def test_config_validation(field, value, code):
    c = cfg(**{field: value})
    L = F.lib()
    st = L.infllm_build_units(ctypes.byref(c), 1, FAKE, 1024, FAKE, 1024, 1024, FAKE, FAKE,
                              FAKE, 1 << 30, None)
    assert st == code
    st = L.infllm_attend(ctypes.byref(c), 1, FAKE, 1024, 0, 0, 64, 1, FAKE, FAKE, 1024, FAKE,
                         FAKE, None, 1024, 0, FAKE, 1 << 30, None)
    assert st == code


def test_build_argument_validation():
    c = cfg()
    L = F.lib()
    call = lambda **kw: L.infllm_build_units(
        ctypes.byref(c), kw.get("batch", 1), kw.get("q", FAKE), kw.get("q_cap", 8192),
        kw.get("k", FAKE), kw.get("kv_cap", 8192), kw.get("n_ctx", 8192), kw.get("rep", FAKE),
        kw.get("repr", FAKE), kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert call(batch=0) == F.INFLLM_ERR_INVALID_ARG
    assert call(n_ctx=0) == F.INFLLM_ERR_INVALID_ARG
    assert call(q_cap=100) == F.INFLLM_ERR_INVALID_ARG
    assert call(kv_cap=100) == F.INFLLM_ERR_INVALID_ARG
    assert call(q=None) == F.INFLLM_ERR_INVALID_ARG
    assert call(k=MISALIGNED) == F.INFLLM_ERR_INVALID_ARG
    assert call(rep=None) == F.INFLLM_ERR_INVALID_ARG
    assert call(repr=MISALIGNED) == F.INFLLM_ERR_INVALID_ARG
    need = F.infllm_workspace_size(c, F.INFLLM_CALL_BUILD, 1, 8192)
    assert need > 0
    assert call(wsb=need - 1) == F.INFLLM_ERR_WORKSPACE
    assert call(ws=None) == F.INFLLM_ERR_WORKSPACE
    # MEAN needs no queries, no rep_idx and no workspace
    cm = cfg(rep_mode=F.INFLLM_REP_MEAN)
    assert F.infllm_workspace_size(cm, F.INFLLM_CALL_BUILD, 1, 8192) == 0


def test_build_range_validation_and_workspace():
    c = cfg()
    L = F.lib()
    U = F.infllm_num_units(c, 8192)             # 63 units
    call = lambda **kw: L.infllm_build_units_range(
        ctypes.byref(c), kw.get("batch", 1), kw.get("q", FAKE), 8192, kw.get("k", FAKE), 8192,
        kw.get("n_ctx", 8192), kw.get("ub", 10), kw.get("ue", 20), kw.get("pool", 64),
        kw.get("rep", FAKE), kw.get("repr", FAKE), kw.get("ws", FAKE), kw.get("wsb", 1 << 30),
        None)
    assert call(ub=-1) == F.INFLLM_ERR_INVALID_ARG
    assert call(ub=21) == F.INFLLM_ERR_INVALID_ARG           # u_end < u_begin
    assert call(ue=U + 1, pool=U + 1) == F.INFLLM_ERR_INVALID_ARG
    assert call(pool=19) == F.INFLLM_ERR_INVALID_ARG         # pool smaller than u_end
    assert call(n_ctx=0) == F.INFLLM_ERR_INVALID_ARG
    assert call(rep=None) == F.INFLLM_ERR_INVALID_ARG
    assert call(repr=MISALIGNED) == F.INFLLM_ERR_INVALID_ARG
    assert call(q=None) == F.INFLLM_ERR_INVALID_ARG
    need = F.infllm_workspace_size(c, F.INFLLM_CALL_BUILD_RANGE, 1, 10)
    assert need > 0
    assert call(wsb=need - 1) == F.INFLLM_ERR_WORKSPACE
    # an empty range succeeds without touching a device
    assert call(ub=5, ue=5, rep=None, repr=None, ws=None, wsb=0) == F.INFLLM_OK
    # range workspace grows with the range, not with the context
    small = F.infllm_workspace_size(c, F.INFLLM_CALL_BUILD_RANGE, 1, 4)
    assert small < need < F.infllm_workspace_size(c, F.INFLLM_CALL_BUILD, 1, 1 << 20)
    assert F.infllm_workspace_size(c, F.INFLLM_CALL_BUILD_RANGE, 1, 0) == 0
    cm = cfg(rep_mode=F.INFLLM_REP_MEAN)
    assert F.infllm_workspace_size(cm, F.INFLLM_CALL_BUILD_RANGE, 1, 10) == 0


def test_varlen_validation():
    c = cfg()
    L = F.lib()
    r = ctypes.byref(c)
    sc = lambda pos: L.infllm_score_units_varlen(r, 2, FAKE, 1000, 0, pos, 1, 1, FAKE, 10, FAKE,
                                                 FAKE, 1 << 30, None)
    assert sc(None) == F.INFLLM_ERR_INVALID_ARG
    assert sc(FAKE + 4) == F.INFLLM_ERR_INVALID_ARG          # not 8-byte aligned
    at = lambda pos, kv_cap=4096, n_chunks=1: L.infllm_attend_varlen(
        r, 2, FAKE, 4096, 0, pos, 512, n_chunks, FAKE, FAKE, kv_cap, FAKE, FAKE, None, 4096, 0,
        FAKE, 1 << 30, None)
    assert at(None) == F.INFLLM_ERR_INVALID_ARG
    assert at(FAKE + 4) == F.INFLLM_ERR_INVALID_ARG
    assert at(FAKE, kv_cap=511) == F.INFLLM_ERR_INVALID_ARG   # no position fits
    assert at(FAKE, n_chunks=9) == F.INFLLM_ERR_INVALID_ARG   # rows beyond q_cap


def test_select_validation_and_workspace():
    c = cfg()
    L = F.lib()
    r = ctypes.byref(c)
    call = lambda **kw: L.infllm_select_units(
        r, 2, FAKE, 1000, 0, 5000, kw.get("pos", None), 1, 1, FAKE, 1023, FAKE, kw.get("sel", FAKE),
        kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert call(sel=None) == F.INFLLM_ERR_INVALID_ARG
    assert call(sel=MISALIGNED) == F.INFLLM_ERR_INVALID_ARG
    assert call(pos=FAKE + 4) == F.INFLLM_ERR_INVALID_ARG
    need = F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT, 2, 0, 1, 1)
    assert need > 0 and F.infllm_workspace_size(c, F.INFLLM_CALL_SCORE, 2, 0, 1, 1) == 0
    assert call(wsb=need - 1) == F.INFLLM_ERR_WORKSPACE
    assert call(ws=None, wsb=0) == F.INFLLM_ERR_WORKSPACE
    # long chunks: the scoring workspace, which already holds the counters
    assert F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT, 2, 0, 512, 3) == \
        F.infllm_workspace_size(c, F.INFLLM_CALL_SCORE, 2, 0, 512, 3)


def test_select_attend_validation_and_workspace():
    c = cfg(top_k=32)
    L = F.lib()
    r = ctypes.byref(c)
    # batch 4 at 128K context: 1,023 units, one position
    call = lambda **kw: L.infllm_select_attend(
        r, 4, FAKE, 300, 0, kw.get("q_pos", 131072), kw.get("pos", None), kw.get("n_pos", 1),
        FAKE, kw.get("U", 1023), FAKE, FAKE, kw.get("kv_cap", 131072 + 256), FAKE,
        kw.get("sel", FAKE), FAKE, None, 300, 0, kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert call(sel=None) == F.INFLLM_ERR_INVALID_ARG
    assert call(sel=MISALIGNED) == F.INFLLM_ERR_INVALID_ARG
    assert call(pos=FAKE + 4) == F.INFLLM_ERR_INVALID_ARG
    assert call(n_pos=0) == F.INFLLM_ERR_INVALID_ARG
    assert call(kv_cap=131072) == F.INFLLM_ERR_INVALID_ARG       # position past the K/V rows
    assert call(U=-1) == F.INFLLM_ERR_INVALID_ARG
    need = F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT_ATTEND, 4, 1023, 1, 1)
    # at least what the two separate calls need, one after the other
    sep = F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT, 4, 0, 1, 1) + \
        F.infllm_workspace_size(c, F.INFLLM_CALL_ATTEND, 4, 0, 1, 1)
    assert need >= sep > 0
    assert call(wsb=need - 1) == F.INFLLM_ERR_WORKSPACE
    assert call(ws=None, wsb=0) == F.INFLLM_ERR_WORKSPACE
    assert call(ws=MISALIGNED) == F.INFLLM_ERR_WORKSPACE
    # one query per chunk only
    assert F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT_ATTEND, 4, 1023, 2, 1) == 0
    # past 2,048 units (separate calls) the size still covers both calls
    big = F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT_ATTEND, 2, 8191, 1, 1)
    assert big >= F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT, 2, 0, 1, 1) + \
        F.infllm_workspace_size(c, F.INFLLM_CALL_ATTEND, 2, 0, 1, 1)


def test_qsum_validation_and_workspace():
    c = cfg()
    L = F.lib()
    r = ctypes.byref(c)
    sc = lambda **kw: L.infllm_score_units_qsum(
        r, 1, kw.get("bq", FAKE), kw.get("nb", 64), kw.get("q_pos", 0), kw.get("L", 512),
        kw.get("nc", 4), FAKE, 60, FAKE, None)
    assert sc(q_pos=100) == F.INFLLM_ERR_INVALID_ARG         # not a multiple of B
    assert sc(L=500) == F.INFLLM_ERR_INVALID_ARG             # chunk not whole blocks
    assert sc(nc=17) == F.INFLLM_ERR_INVALID_ARG             # past the last block
    assert sc(bq=None) == F.INFLLM_ERR_INVALID_ARG
    assert sc(nb=0) == F.INFLLM_ERR_INVALID_ARG
    bd = lambda **kw: L.infllm_build_units_qsum(
        r, 1, kw.get("q", FAKE), 8192, FAKE, 8192, 8192, FAKE, FAKE, kw.get("bq", FAKE),
        FAKE, kw.get("wsb", 1 << 30), None)
    assert bd(bq=None) == F.INFLLM_ERR_INVALID_ARG
    assert bd(q=None) == F.INFLLM_ERR_INVALID_ARG
    need = F.infllm_workspace_size(c, F.INFLLM_CALL_BUILD_QSUM, 1, 8192)
    assert need > 0
    assert bd(wsb=need - 1) == F.INFLLM_ERR_WORKSPACE
    cm = cfg(rep_mode=F.INFLLM_REP_MEAN)
    assert F.infllm_workspace_size(cm, F.INFLLM_CALL_BUILD_QSUM, 1, 8192) == 0


def test_score_topk_attend_validation():
    c = cfg()
    L = F.lib()
    r = ctypes.byref(c)
    # score: rows beyond q_cap, negative offsets, misaligned outputs
    assert L.infllm_score_units(r, 1, FAKE, 1000, 600, 600, 512, 1, FAKE, 10, FAKE, None, 0,
                                None) == F.INFLLM_ERR_INVALID_ARG
    assert L.infllm_score_units(r, 1, FAKE, 1000, -1, 0, 512, 1, FAKE, 10, FAKE, None, 0,
                                None) == F.INFLLM_ERR_INVALID_ARG
    assert L.infllm_score_units(r, 1, FAKE, 1000, 0, 0, 512, 1, FAKE, 10, MISALIGNED, None, 0,
                                None) == F.INFLLM_ERR_INVALID_ARG
    assert L.infllm_score_units(r, 1, FAKE, 1000, 0, 0, 0, 1, FAKE, 10, FAKE, None, 0,
                                None) == F.INFLLM_ERR_INVALID_ARG
    # topk: missing outputs
    assert L.infllm_topk_units(r, 1, 1, FAKE, 10, None, None, 0, None) == F.INFLLM_ERR_INVALID_ARG
    assert L.infllm_topk_units(r, 1, 0, FAKE, 10, FAKE, None, 0, None) == F.INFLLM_ERR_INVALID_ARG
    # top_k = 0 is a no-op that succeeds without touching a device
    c0 = cfg(top_k=0)
    assert L.infllm_topk_units(ctypes.byref(c0), 1, 1, FAKE, 10, None, None, 0, None) == F.INFLLM_OK
    # attend: K/V must hold every query position, output rows within out_cap
    a = lambda **kw: L.infllm_attend(
        r, 1, FAKE, kw.get("q_cap", 4096), kw.get("q_off", 0), kw.get("q_pos", 0),
        kw.get("L", 512), kw.get("nc", 1), FAKE, FAKE, kw.get("kv_cap", 4096), kw.get("sel", FAKE),
        FAKE, None, kw.get("out_cap", 4096), kw.get("out_off", 0), FAKE, 1 << 30, None)
    assert a(q_pos=3600) == F.INFLLM_ERR_INVALID_ARG
    assert a(q_off=3600) == F.INFLLM_ERR_INVALID_ARG
    assert a(out_off=3600) == F.INFLLM_ERR_INVALID_ARG
    assert a(sel=None) == F.INFLLM_ERR_INVALID_ARG
    assert a(L=0) == F.INFLLM_ERR_INVALID_ARG
    assert a(q_pos=-5) == F.INFLLM_ERR_INVALID_ARG


def test_attend_workspace_sizing():
    c = cfg()
    # decode: one position per (sequence, KV head) needs split-K partials
    ws_dec = F.infllm_workspace_size(c, F.INFLLM_CALL_ATTEND, 4, 0, 1, 1)
    assert ws_dec > 0 and ws_dec % 4 == 0
    L = F.lib()
    st = L.infllm_attend(ctypes.byref(c), 4, FAKE, 1, 0, 131072, 1, 1, FAKE, FAKE, 131328, FAKE,
                         FAKE, None, 1, 0, FAKE, ws_dec - 1, None)
    assert st == F.INFLLM_ERR_WORKSPACE
