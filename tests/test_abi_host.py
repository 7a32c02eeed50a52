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
    assert len(names) == 24
    assert set(names) == set(F.EXPORTED)
    L = F.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.infllm_abi_version() == 2


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
    assert need > 0
    assert call(wsb=need - 1) == F.INFLLM_ERR_WORKSPACE
    assert call(ws=None, wsb=0) == F.INFLLM_ERR_WORKSPACE
    assert call(ws=MISALIGNED) == F.INFLLM_ERR_WORKSPACE
    # one query per chunk only
    assert F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT_ATTEND, 4, 1023, 2, 1) == 0


# (batch, KV heads, G, units, k_m, positions)
STEP_SHAPES = [(4, 8, 4, 1023, 32, 1), (2, 8, 4, 8191, 32, 1), (1, 8, 4, 511, 32, 1),
               (8, 8, 4, 8191, 32, 1), (8, 8, 4, 1023, 32, 16), (4, 8, 8, 1023, 32, 64),
               (1, 2, 4, 18, 4, 1), (1, 8, 4, 2047, 256, 1), (1, 8, 4, 4095, 256, 1),
               (2, 1, 8, 16384, 32, 1), (2, 1, 8, 16385, 32, 1), (1, 1, 1, 1, 1, 1),
               (64, 8, 4, 1023, 32, 1), (1, 8, 4, 1023, 300, 1)]


@pytest.mark.parametrize("b,Hkv,G,U,k_m,n_pos", STEP_SHAPES)
def test_step_plan(b, Hkv, G, U, k_m, n_pos):
    """The one-launch decode step's plan: scoring workgroups cover the units
    exactly once, at least one attention workgroup per row has no slice, at
    most 64 attention workgroups per row (plus the selector), every score
    of a row is a candidate (rows with more take the two calls unless the
    split count is set by hand), and the workspace holds the row state, the
    candidates and every split's partial rows.  Large batches and many
    positions stay in one launch even when the grid exceeds what the chip
    holds at once (the waits do not depend on residency)."""
    c = cfg(n_q_heads=G * Hkv, n_kv_heads=Hkv, top_k=k_m)
    if k_m > 256:
        assert F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT_ATTEND, b, U, 1, n_pos) == 0
        return
    p = F.infllm_step_plan(c, b, U, n_pos)
    total = F.infllm_workspace_size(c, F.INFLLM_CALL_SELECT_ATTEND, b, U, 1, n_pos)
    c0, c1, t = F.infllm_workspace_layout(c, F.INFLLM_CALL_SELECT_ATTEND, b, U, 1, n_pos)
    rows = b * Hkv * n_pos
    assert t == total > 0 and c0 == 256 and c1 - c0 >= 65536 and total >= c1
    if not p["fused"]:
        # more scores in a row than one search takes at the coarsest slices
        assert -(-U // 256) * 256 > 2048 or U > 2048
        return
    N, S, up, C = p["n_splits"], p["s_score"], p["units_per"], p["cand"]
    assert 2 <= N <= 64 and 1 <= S < N
    assert up in (64, 128, 192, 256) and (S - 1) * up < U <= S * up
    assert C == up and S * C <= 2048
    assert p["w_score"] >= 0 and p["w_unit"] >= 0 and p["w_score"] + p["w_unit"] >= 1
    assert c1 - c0 >= 80 * rows
    d, Hq = 128, G * Hkv
    assert total >= c1 + rows * S * C * 8 + N * b * Hq * n_pos * (d * 4 + 8)



@pytest.mark.parametrize("b,Hkv,U,n_pos,per_cu", [
    (4, 8, 1023, 1, 2),     # 128K decode: 153 MB per step, two workgroups per CU
    (1, 8, 511, 1, 1),      # Mistral 64K decode: 36 MB, one per CU
    (1, 4, 1023, 1, 1),     # a light step: one per CU (64 workgroups a row)
    (8, 8, 1023, 1, 3),     # 306 MB: three per CU (the most resident at once)
    (2, 8, 2047, 2, 3)])    # 171 MB: three per CU
def test_step_plan_grid(b, Hkv, U, n_pos, per_cu):
    """The one-launch decode step's grid is a whole number of workgroups per
    CU of the MI355X's 256, one to three, about one per CU for every 64 MiB
    the step moves: a grid with some CUs holding one workgroup more than
    others ends when those do.  (Rows of fewer than 4 rows a call stop at
    64 attention workgroups a row.)"""
    c = cfg(n_q_heads=4 * Hkv, n_kv_heads=Hkv, top_k=32)
    p = F.infllm_step_plan(c, b, U, n_pos)
    assert p["fused"] == 1
    rows = b * Hkv * n_pos
    assert (p["n_splits"] + 1) * rows == 256 * per_cu

def test_step_plan_rope():
    """With positions inside the working context the one-launch step holds
    at most two workgroups per CU (its turned keys take the registers of a
    third), and takes the two calls with 8 query heads per KV head or
    head_dim 64."""
    for b, Hkv, U, per_cu in [(8, 8, 1023, 2), (4, 8, 1023, 2), (1, 8, 511, 1)]:
        c = cfg(n_q_heads=4 * Hkv, n_kv_heads=Hkv, top_k=32, rope_theta=500000.0)
        p = F.infllm_step_plan(c, b, U, 1)
        assert p["fused"] == 1 and (p["n_splits"] + 1) * b * Hkv == 256 * per_cu
    for G, d in [(8, 128), (4, 64)]:
        c = cfg(n_q_heads=G * 2, n_kv_heads=2, head_dim=d, top_k=8, rope_theta=10000.0)
        assert F.infllm_step_plan(c, 1, 300, 1)["fused"] == 0


def test_workspace_counter_regions():
    """Every call kind keeps its counters in [256, 256 + region) with a
    region of at least 64 KiB, and its data after it: a zero-filled
    workspace may serve calls of other kinds and shapes whose counters fit
    64 KiB without a counter landing on another call's data."""
    c = cfg()
    cases = [(F.INFLLM_CALL_SCORE, 1, 0, 512, 64), (F.INFLLM_CALL_SELECT, 4, 0, 1, 1),
             (F.INFLLM_CALL_SELECT, 1, 0, 512, 64), (F.INFLLM_CALL_ATTEND, 4, 0, 1, 1),
             (F.INFLLM_CALL_ATTEND, 1, 0, 1, 4), (F.INFLLM_CALL_ATTEND, 1, 0, 512, 1),
             (F.INFLLM_CALL_SELECT_ATTEND, 4, 1023, 1, 1),
             (F.INFLLM_CALL_SELECT_ATTEND, 2, 8191, 1, 1),
             (F.INFLLM_CALL_SELECT_ATTEND, 8, 4095, 1, 8)]
    for call, b, n, L, nc in cases:
        c0, c1, total = F.infllm_workspace_layout(c, call, b, n, L, nc)
        assert total == F.infllm_workspace_size(c, call, b, n, L, nc)
        assert total > 0 and c0 == 256 and c1 - c0 == 65536 and total >= c1, (call, b, n, L, nc)
    # a step whose counters need more than 64 KiB: its own, larger region
    c0, c1, total = F.infllm_workspace_layout(c, F.INFLLM_CALL_SELECT_ATTEND, 8, 1023, 1, 256)
    assert c0 == 256 and c1 - c0 >= 16 * 8 * 8 * 256 > 65536
    # calls without counters
    assert F.infllm_workspace_layout(c, F.INFLLM_CALL_SCORE, 4, 0, 1, 1) == (0, 0, 0)
    # the single-pass build: flags of the published block sums (one int per
    # block and a counter per (sequence, KV head)) in the region, the sums
    # after it; 64 KiB up to 16K blocks per head group at 8 KV heads
    for call, b, n, n_units in ((F.INFLLM_CALL_BUILD, 1, 8192, 63),
                                (F.INFLLM_CALL_BUILD, 2, 1 << 20, 8191),
                                (F.INFLLM_CALL_BUILD_RANGE, 4, 1, 1)):
        c0, c1, total = F.infllm_workspace_layout(c, call, b, n, 0, 0)
        assert total == F.infllm_workspace_size(c, call, b, n, 0, 0)
        nbl = n_units + 4096 // 128 + 1
        assert c0 == 256 and c1 - c0 == max(65536, -(-(b * 8 * (nbl + 1) * 4) // 256) * 256)
        assert total >= c1 + b * 8 * nbl * 4 * 128 * 8, (call, b, n)   # 4 quarter prefixes
    mean = cfg(rep_mode=F.INFLLM_REP_MEAN)
    assert F.infllm_workspace_layout(mean, F.INFLLM_CALL_BUILD, 1, 8192, 0, 0) == (0, 0, 0)


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


def test_static_scratch_limits():
    """infllm_select_attend_static refuses, before any device call, a step
    whose workspace exceeds the library's 16 MiB scratch array or whose
    counters exceed the fixed 64 KiB counter region, and validates its
    arguments like infllm_select_attend."""
    c = cfg(top_k=32)
    L = F.lib()
    r = ctypes.byref(c)

    def call(batch, n_pos, U=1023, sel=FAKE):
        return L.infllm_select_attend_static(r, batch, FAKE, 1 << 20, 0, 131072, None, n_pos, FAKE,
                                             U, FAKE, FAKE, 131072 + 4096, FAKE, sel, FAKE, None,
                                             1 << 20, 0, None)
    # 64 x 8 x 64 rows: counters beyond the region (and partials beyond 16 MiB)
    big = F.infllm_workspace_layout(c, F.INFLLM_CALL_SELECT_ATTEND, 64, 1023, 1, 64)
    assert big[1] - big[0] > 65536 or big[2] > (16 << 20)
    assert call(64, 64) == F.INFLLM_ERR_WORKSPACE
    assert call(4, 1, sel=None) == F.INFLLM_ERR_INVALID_ARG
    assert call(0, 1) == F.INFLLM_ERR_INVALID_ARG


# ------------------------------------------------------------------ unit cache
def test_cache_state_size():
    c = cfg()
    # header 256 B; slot_of rows x U int32, unit_of rows x C int32, stamp rows x C int64,
    # each rounded up to 256 B
    def want(rows, U, C):
        r = lambda x: (x + 255) // 256 * 256
        return 256 + r(rows * U * 4) + r(rows * C * 4) + r(rows * C * 8)
    assert F.infllm_cache_state_size(c, 2, 8191, 64) == want(16, 8191, 64)
    assert F.infllm_cache_state_size(c, 1, 1, 1) == want(8, 1, 1)
    assert F.infllm_cache_state_size(c, 0, 10, 10) == 0
    assert F.infllm_cache_state_size(c, 1, 0, 10) == 0
    assert F.infllm_cache_state_size(c, 1, 65537, 10) == 0      # above the unit limit
    assert F.infllm_cache_state_size(c, 1, 100, 1025) == 0      # above the slot limit


def test_cache_fetch_host_checks():
    """Rejections before anything is enqueued (fake, aligned device pointers)."""
    L = F.lib()
    P = 1 << 20       # a 16-byte aligned stand-in address; never dereferenced
    c = cfg(top_k=32)
    U, C = 1000, 64
    host_cap = (U + 1) * 128

    def fetch(cfg_=c, n_pos=1, U_=U, step=1, host_cap_=host_cap, C_=C, sel=P, kh=P, state=P):
        return L.infllm_cache_fetch(ctypes.byref(cfg_), 2, n_pos, sel, U_, step, kh, P, host_cap_,
                                    P, P, C_, state, None)
    assert fetch(n_pos=3) == F.INFLLM_ERR_INVALID_ARG        # 3 x 32 selections > 64 slots
    assert fetch(step=0) == F.INFLLM_ERR_INVALID_ARG
    assert fetch(host_cap_=host_cap - 1) == F.INFLLM_ERR_INVALID_ARG
    assert fetch(kh=None) == F.INFLLM_ERR_INVALID_ARG
    assert fetch(kh=P + 8) == F.INFLLM_ERR_INVALID_ARG        # misaligned
    assert fetch(state=None) == F.INFLLM_ERR_INVALID_ARG
    assert fetch(sel=None) == F.INFLLM_ERR_INVALID_ARG
    assert fetch(U_=70000, host_cap_=(70001) * 128) == F.INFLLM_ERR_UNSUPPORTED
    assert fetch(C_=2000, n_pos=1) == F.INFLLM_ERR_UNSUPPORTED
    # k_m = 0: nothing to fetch, nothing enqueued
    assert fetch(cfg_=cfg(top_k=0), sel=None) == F.INFLLM_OK


def test_attend_cached_host_checks():
    L = F.lib()
    P = 1 << 20
    c = cfg()
    W, n_init = 4096, 128

    def att(cfg_=c, n_pos=1, local_cap=n_init + W, ctx_cap=10000, q_pos=5000, ws_bytes=1 << 30,
            state=P):
        return L.infllm_attend_cached(ctypes.byref(cfg_), 1, P, n_pos, 0, q_pos, None, n_pos, P,
                                      P, local_cap, ctx_cap, P, 100, P, P, 64, state, P, None,
                                      n_pos, 0, P, ws_bytes, None)
    assert att(local_cap=n_init + W - 1) == F.INFLLM_ERR_INVALID_ARG     # ring too short
    assert att(n_pos=4, local_cap=n_init + W + 2) == F.INFLLM_ERR_INVALID_ARG
    assert att(cfg_=cfg(rope_theta=10000.0)) == F.INFLLM_ERR_UNSUPPORTED
    assert att(q_pos=9999, n_pos=2, local_cap=n_init + W + 1) == F.INFLLM_ERR_INVALID_ARG
    assert att(state=None) == F.INFLLM_ERR_INVALID_ARG
    assert att(ws_bytes=0) == F.INFLLM_ERR_WORKSPACE
