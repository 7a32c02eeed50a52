"""GPU parity: every C-ABI stage against the fp64 oracle on the same seeded
inputs, at sizes the oracle finishes in seconds (several tiles, ragged
tails), plus edge cases.  Stage-isolated: each stage gets identical inputs on
both sides; the full pipeline is compared stage by stage on the GPU's own
upstream outputs."""
import numpy as np
import pytest
import torch

from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth
from gpu_helpers import (assert_close, cfg_of, check_rep_idx, check_selection, gpu_attend,
                         gpu_build, gpu_score, gpu_topk, tolerance)

pytestmark = pytest.mark.gpu

LL = synth.WORKLOADS["llama3_8b_32k_encode"]
CASES = {
    # bf16, G=4, d=128, W a multiple of B, ragged context (not a multiple of B)
    "bf16_g4": LL.replace(n_ctx=3136, n_q_heads=8, n_kv_heads=2, window=512, top_k=4, chunk=256),
    # fp32, G=1, d=64, sinks not a multiple of B (partial unit 0), planted block
    "f32_g1": synth.WORKLOADS["tiny_f32"].replace(n_ctx=2048),
    # bf16, G=8, W not a multiple of B, sinks 100, chunk 192
    "bf16_g8_ragged": LL.replace(n_ctx=2500, n_q_heads=8, n_kv_heads=1, window=300, n_init=100,
                                 top_k=5, chunk=192),
    # bf16, mean-of-keys units, clustered keys
    "bf16_mean": synth.WORKLOADS["mistral_7b_64k_mean"].replace(
        n_ctx=3072, n_q_heads=8, n_kv_heads=2, window=512, top_k=6, chunk=256, decode_steps=0),
    # bf16, G=2, d=64
    "bf16_g2_d64": LL.replace(n_ctx=2304, n_q_heads=4, n_kv_heads=2, head_dim=64, window=256,
                              top_k=3, chunk=128, scale=0.125),
    # bf16, G=4, entries of std 1: logits of order 1, so the softmax weights
    # (not only which keys are attended) are checked on the MFMA path
    "bf16_g4_unit": LL.replace(n_ctx=2560, n_q_heads=8, n_kv_heads=2, window=384, top_k=4,
                               chunk=256, scale=1.0),
    # bf16, G=4, 2 sequences x 8 KV heads x 17 blocks (the last one partial):
    # a grid large enough for the build with block query sums to take the
    # single pass
    "bf16_g4_b2": LL.replace(n_ctx=2112, batch=2, n_q_heads=32, n_kv_heads=8, window=512,
                             top_k=4, chunk=256),
}


@pytest.fixture(scope="module")
def data():
    cache = {}

    def get(name):
        if name not in cache:
            w = CASES[name]
            inp = synth.make_inputs(w)
            dev = {k: (v.cuda() if isinstance(v, torch.Tensor) and k != "planted_units" else v)
                   for k, v in inp.items()}
            cache[name] = (w, inp, dev)
        return cache[name]
    return get


def oracle_build(orc, w, inp):
    return orc.build_units_all(inp["q"], inp["k"], w.n_ctx, B=w.block, n_init=w.n_init,
                               W=w.window, r_k=w.rep_k, mode=w.rep_mode)


@pytest.mark.parametrize("name", list(CASES))
def test_build_parity(orc, data, name):
    w, inp, dev = data(name)
    cfg = cfg_of(w)
    rep_g, repr_g = gpu_build(cfg, dev["q"], dev["k"], w.n_ctx)
    torch.cuda.synchronize()
    rep_o, repr_o, ks_o = oracle_build(orc, w, inp)
    rg = repr_g.cpu().numpy()
    if w.rep_mode == "mean":
        np.testing.assert_array_equal(rg, repr_o.astype(np.float32))
        return
    ex = check_rep_idx(rep_g.cpu().numpy(), rep_o, ks_o, w.block, w.n_init)
    assert len(ex) <= max(2, rep_o.shape[2] // 50)
    same = np.all(rep_g.cpu().numpy() == rep_o, axis=-1)
    # same representatives -> the fp64 sum rounded once: bit-identical
    np.testing.assert_array_equal(rg[same], repr_o.astype(np.float32)[same])


def build_rows_fallback_case(orc, name):
    """test_build_parity for one case on a fresh workspace; returns the
    workspace's count of units that summed their window's rows themselves
    (header word 2)."""
    w = CASES[name]
    inp = synth.make_inputs(w)
    cfg = cfg_of(w)
    q, k = inp["q"].cuda(), inp["k"].cuda()
    b, U = w.batch, F.infllm_num_units(cfg, w.n_ctx)
    rep = torch.empty((b, w.n_kv_heads, U, w.rep_k), dtype=torch.int32, device="cuda")
    repr_ = torch.empty((b, w.n_kv_heads, U, w.head_dim), dtype=torch.float32, device="cuda")
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD, b, w.n_ctx)
    F.infllm_build_units(cfg, q, k, w.n_ctx, rep, repr_, ws)
    torch.cuda.synchronize()
    rep_o, repr_o, ks_o = oracle_build(orc, w, inp)
    ex = check_rep_idx(rep.cpu().numpy(), rep_o, ks_o, w.block, w.n_init)
    assert len(ex) <= max(2, rep_o.shape[2] // 50)
    same = np.all(rep.cpu().numpy() == rep_o, axis=-1)
    np.testing.assert_array_equal(repr_.cpu().numpy()[same], repr_o.astype(np.float32)[same])
    return int(ws[8:12].view(torch.int32)[0])


def test_build_from_rows():
    """INFLLM_BUILD_SPIN=0: every unit that would take the published block
    sums of the blocks after it sums its window's query rows itself instead
    (the path a unit takes when those sums are late): the same selection as
    the oracle, and the header counts the units that did."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys\n"
            "sys.path[:0] = [%r, %r]\n"
            "from oracle import oracle as orc\n"
            "import test_gpu_parity as t\n"
            "for name in ('bf16_g4', 'f32_g1', 'bf16_g2_d64', 'bf16_g4_unit'):\n"
            "    print('case', name, flush=True)\n"
            "    print('from rows', name, t.build_rows_fallback_case(orc, name), flush=True)\n"
            "print('ok', flush=True)\n") % (here, os.path.dirname(here))
    env = dict(os.environ, INFLLM_BUILD_SPIN="0")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
    for line in r.stdout.splitlines():
        if line.startswith("from rows"):
            name, n = line.split()[2], int(line.split()[3])
            w = CASES[name]
            U = F.infllm_num_units(cfg_of(w), w.n_ctx)
            assert 0 < n <= w.batch * w.n_kv_heads * U, line


def check_units(orc, w, inp, n_ctx, u_lo, u_hi, rep_g, repr_g):
    """GPU rows u_lo .. u_hi-1 (rep_g / repr_g: [b, H_kv, u_hi-u_lo, .]) against
    the oracle's build of a context of n_ctx tokens, per (batch, KV head)."""
    G, B = w.group, w.block
    exemptions = 0
    for bi in range(w.batch):
        for h in range(w.n_kv_heads):
            k = inp["k"][bi, h, :n_ctx]
            if w.rep_mode == "mean":
                repr_o = orc.build_mean(k, B, w.n_init, u_lo, u_hi)
                np.testing.assert_array_equal(repr_g[bi, h], repr_o.astype(np.float32))
                continue
            rep_o, repr_o, ks_o = orc.build_tokens(inp["q"][bi, h * G:(h + 1) * G, :n_ctx], k,
                                                   n_ctx, B, w.n_init, w.window, w.rep_k,
                                                   u_lo, u_hi)
            for i in range(u_hi - u_lo):
                if np.array_equal(rep_g[bi, h, i], rep_o[i]):
                    np.testing.assert_array_equal(repr_g[bi, h, i], repr_o[i].astype(np.float32))
                    continue
                start = (u_lo + i + w.n_init // B) * B
                by_pos = {start + s: ks_o[i, s] for s in range(B) if np.isfinite(ks_o[i, s])}
                exemptions += check_selection(rep_g[bi, h, i], rep_o[i], by_pos)
    assert exemptions <= max(2, w.batch * w.n_kv_heads * (u_hi - u_lo) // 50)


def range_pool(cfg, w, pool):
    """A unit pool of `pool` rows filled with values no build writes."""
    repr_ = torch.full((w.batch, w.n_kv_heads, pool, w.head_dim), float("nan"), device="cuda")
    rep = None
    if w.rep_mode == "tokens":
        rep = torch.full((w.batch, w.n_kv_heads, pool, w.rep_k), -7, dtype=torch.int32,
                         device="cuda")
    return rep, repr_


@pytest.mark.parametrize("name", list(CASES))
def test_build_range_streaming(orc, data, name):
    """Units appended to a pool as their keys leave the local window, one
    range call per step at the context reached so far; the units still in
    the window at the end are built at the final context.  The pool equals
    the oracle's build of the final context: a closed unit's windows lie
    inside every later context."""
    w, inp, dev = data(name)
    cfg = cfg_of(w)
    B = w.block
    U = F.infllm_num_units(cfg, w.n_ctx)
    rep, repr_ = range_pool(cfg, w, U + 3)
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_RANGE, w.batch, U, device="cuda")
    rng = np.random.default_rng(11)
    done, n, calls = 0, w.n_init + w.window + 1, 0
    while n < w.n_ctx:
        closed = done
        while closed < U and orc.unit_keys(closed, B, w.n_init)[1] <= n - w.window:
            closed += 1
        F.infllm_build_units_range(cfg, dev["q"], dev["k"], n, done, closed, rep, repr_, ws)
        done, calls = closed, calls + 1
        n += int(rng.integers(1, 3 * B))
    F.infllm_build_units_range(cfg, dev["q"], dev["k"], w.n_ctx, done, U, rep, repr_, ws)
    torch.cuda.synchronize()
    assert calls >= 5 and 0 < done < U
    rg = repr_.cpu().numpy()
    assert np.isnan(rg[:, :, U:]).all()
    repg = None
    if rep is not None:
        repg = rep.cpu().numpy()
        assert (repg[:, :, U:] == -7).all()
        repg = repg[:, :, :U]
    check_units(orc, w, inp, w.n_ctx, 0, U, repg, rg[:, :, :U])


@pytest.mark.parametrize("name", list(CASES))
def test_build_range_truncated(orc, data, name):
    """A range that ends in units whose windows run past the current
    position (scores truncated there), written at its rows of a larger pool
    with every other row untouched; an empty range writes nothing."""
    w, inp, dev = data(name)
    cfg = cfg_of(w)
    n_mid = w.n_ctx - 333
    Um = F.infllm_num_units(cfg, n_mid)
    lo = Um // 3
    rep, repr_ = range_pool(cfg, w, Um + 5)
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_RANGE, w.batch, Um - lo, device="cuda")
    F.infllm_build_units_range(cfg, dev["q"], dev["k"], n_mid, lo, Um, rep, repr_, ws)
    F.infllm_build_units_range(cfg, dev["q"], dev["k"], n_mid, 2, 2, rep, repr_, ws)
    torch.cuda.synchronize()
    rg = repr_.cpu().numpy()
    assert np.isnan(rg[:, :, :lo]).all() and np.isnan(rg[:, :, Um:]).all()
    repg = None
    if rep is not None:
        repg = rep.cpu().numpy()
        assert (repg[:, :, :lo] == -7).all() and (repg[:, :, Um:] == -7).all()
        repg = repg[:, :, lo:Um]
    check_units(orc, w, inp, n_mid, lo, Um, repg, rg[:, :, lo:Um])


@pytest.mark.parametrize("name", ["bf16_g4", "bf16_g8_ragged"])
def test_build_nan_queries_stay_in_rows(data, name):
    """Query rows holding NaN give some keys NaN scores: every unit still
    keeps exactly r_k distinct keys of its own (NaN scores rank behind every
    number), and nothing is written outside the range's rows of the pool --
    for the range build, the full build and the build with block query sums."""
    w, inp, dev = data(name)
    cfg = cfg_of(w)
    q = dev["q"].clone()
    q[:, :, 700:705] = float("nan")
    q[:, 1, 1900] = float("nan")
    U = F.infllm_num_units(cfg, w.n_ctx)
    B, n_init, r_k = w.block, w.n_init, w.rep_k

    def check(rep, lo, hi):
        repg = rep.cpu().numpy()
        assert (repg[:, :, :lo] == -7).all() and (repg[:, :, hi:] == -7).all()
        for u in range(lo, hi):
            first = max((u + n_init // B) * B, n_init)
            ids = repg[:, :, u].reshape(-1, r_k)
            for row in ids:
                assert len(set(row.tolist())) == r_k, (u, row)
                assert ((row >= first) & (row < (u + n_init // B + 1) * B)).all(), (u, row)

    rep, repr_ = range_pool(cfg, w, U + 3)
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_RANGE, w.batch, U - 2, device="cuda")
    F.infllm_build_units_range(cfg, q, dev["k"], w.n_ctx, 2, U, rep, repr_, ws)
    torch.cuda.synchronize()
    check(rep, 2, U)
    rep, repr_ = range_pool(cfg, w, U)
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD, w.batch, w.n_ctx, device="cuda")
    F.infllm_build_units(cfg, q, dev["k"], w.n_ctx, rep, repr_, ws)
    torch.cuda.synchronize()
    check(rep, 0, U)
    rep, repr_ = range_pool(cfg, w, U)
    nb = (w.n_ctx + B - 1) // B
    bq = torch.empty((w.batch, w.n_kv_heads, nb, w.head_dim), dtype=torch.float64, device="cuda")
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_QSUM, w.batch, w.n_ctx, device="cuda")
    F.infllm_build_units_qsum(cfg, q, dev["k"], w.n_ctx, rep, repr_, bq, ws)
    torch.cuda.synchronize()
    check(rep, 0, U)


@pytest.mark.parametrize("name", list(CASES))
def test_score_and_topk_parity(orc, data, name):
    w, inp, dev = data(name)
    cfg = cfg_of(w)
    U = orc.num_units(w.n_ctx, w.block, w.n_init)
    gen = torch.Generator().manual_seed(7)
    repr32 = (torch.randn((w.batch, w.n_kv_heads, U, w.head_dim), generator=gen)).float()
    n_chunks = w.n_ctx // w.chunk
    scores = gpu_score(cfg, dev["q"], 0, 0, w.chunk, n_chunks, repr32.cuda())
    # the same chunks one call at a time give bit-identical scores
    s1 = gpu_score(cfg, dev["q"], w.chunk, w.chunk, w.chunk, 1, repr32.cuda())
    torch.cuda.synchronize()
    assert torch.equal(scores[:, :, 1:2], s1)
    sg = scores.cpu().numpy()
    sel_g = gpu_topk(cfg, scores).cpu().numpy()
    G = w.group
    for c in range(n_chunks):
        t0 = c * w.chunk
        e = orc.num_eligible(t0 + w.chunk - 1, U, w.block, w.n_init, w.window)
        assert F.infllm_num_eligible(cfg, t0 + w.chunk - 1, U) == e
        for bi in range(w.batch):
            for h in range(w.n_kv_heads):
                so = orc.score_units(inp["q"][bi, h * G:(h + 1) * G, t0:t0 + w.chunk],
                                     repr32[bi, h].double().numpy(), e)
                fin = np.isfinite(so)
                assert (np.isfinite(sg[bi, h, c]) == fin).all()
                np.testing.assert_allclose(sg[bi, h, c][fin], so[fin], rtol=1e-6,
                                           atol=1e-6 * np.abs(so[fin]).max(initial=1.0))
                # top-k on the GPU's fp32 scores: exact against the oracle on
                # the same (widened) values
                so32 = sg[bi, h, c].astype(np.float64)
                assert sel_g[bi, h, c].tolist() == orc.topk(so32, e, w.top_k).tolist()
                # and within the near-tie rule of the oracle's own fp64 scores
                check_selection(sel_g[bi, h, c], orc.topk(so, e, w.top_k), so)


@pytest.mark.parametrize("U,k_m,ties", [(1, 4, False), (7, 3, True), (255, 16, True),
                                        (1023, 32, False), (8191, 32, True), (8191, 256, False),
                                        (40, 64, False), (300, 1, True), (2048, 32, True),
                                        (2049, 5, True), (16000, 32, True), (20000, 8, False),
                                        (64, 64, False), (4096, 256, True), (40000, 16, True),
                                        (1500, 32, True), (600, 8, False), (8193, 32, False),
                                        (12000, 16, True)])
def test_topk_exact(orc, U, k_m, ties):
    gen = torch.Generator().manual_seed(U * 131 + k_m)
    # 1500 and 600 units: enough problems (2 x 2 x 256) for the one-wave variant
    nc = 256 if U in (1500, 600) else 3
    if ties:
        s = torch.randint(-6, 6, (2, 2, nc, U), generator=gen).float() * 0.5
    else:
        s = torch.randn((2, 2, nc, U), generator=gen)
    s[..., U - U // 5:] = -float("inf")                       # an ineligible tail
    s[1, 1, 2] = -float("inf")                                # nothing eligible
    s[0, 1, 1, :3] = torch.tensor([0.0, -0.0, 0.0])[:min(3, U)]
    cfg = F.make_config(n_q_heads=4, n_kv_heads=2, head_dim=128, block=128, n_init=128,
                        window=512, rep_k=4, top_k=k_m)
    sel = gpu_topk(cfg, s.cuda()).cpu().numpy()
    for idx in np.ndindex(s.shape[:3]):
        row = s[idx].double().numpy()
        e = int(np.argmax(~np.isfinite(row))) if not np.isfinite(row).all() else U
        assert sel[idx].tolist() == orc.topk(row, e, k_m).tolist(), idx


def _oracle_selection(orc, w, inp, t0, L, repr_o):
    _, sel, e = orc.select_all(inp["q"][:, :, t0:t0 + L], t0, repr_o, B=w.block, n_init=w.n_init,
                               W=w.window, k_m=w.top_k)
    return sel


@pytest.mark.parametrize("name", list(CASES))
def test_attend_chunks_parity(orc, data, name):
    """Chunked encoding: every chunk in one call (per-chunk selections)."""
    w, inp, dev = data(name)
    cfg = cfg_of(w)
    _, repr_o, _ = oracle_build(orc, w, inp)
    n_chunks = w.n_ctx // w.chunk
    sels = np.stack([_oracle_selection(orc, w, inp, c * w.chunk, w.chunk, repr_o)
                     for c in range(n_chunks)], axis=2)            # [b, H_kv, nc, k_m]
    out, lse = gpu_attend(cfg, dev["q"], 0, 0, w.chunk, n_chunks, dev["k"], dev["v"],
                          torch.from_numpy(sels).cuda())
    torch.cuda.synchronize()
    # oracle on a sample of chunks: first, one in the middle, the last
    for c in sorted({0, n_chunks // 2, n_chunks - 1}):
        t0 = c * w.chunk
        o_ref, l_ref = orc.attend_all(inp["q"][:, :, t0:t0 + w.chunk], t0, inp["k"], inp["v"],
                                      sels[:, :, c], B=w.block, n_init=w.n_init, W=w.window)
        tol = tolerance(inp["q"].dtype, o_ref)
        assert_close(out[:, :, t0:t0 + w.chunk], o_ref, tol, "%s chunk %d out" % (name, c))
        assert_close(lse[:, :, t0:t0 + w.chunk], l_ref, 1e-3, "%s chunk %d lse" % (name, c))


@pytest.mark.parametrize("name", ["bf16_g4", "f32_g1", "bf16_g8_ragged"])
def test_attend_edge_cases(orc, data, name):
    w, inp, dev = data(name)
    U = orc.num_units(w.n_ctx, w.block, w.n_init)
    G = w.group
    # (a) k_m = 0: sinks + window only; (b) every unit selected: dense causal;
    # (c) a ragged chunk of 37 queries straddling the first eligible unit;
    # (d) decode-like single positions, including t < n_init
    cases = [("no_units", cfg_of(w, top_k=0), np.zeros((w.batch, w.n_kv_heads, 1, 0), np.int32),
              w.n_ctx - 100, 100),
             ("all_units", cfg_of(w, top_k=min(U, 256)),
              np.broadcast_to(np.arange(min(U, 256), dtype=np.int32),
                              (w.batch, w.n_kv_heads, 1, min(U, 256))).copy(), w.n_ctx - 64, 64),
             ("ragged", cfg_of(w), None, w.window + w.n_init - 20, 37),
             ("early", cfg_of(w), None, 0, 1),
             ("late_single", cfg_of(w), None, w.n_ctx - 1, 1)]
    # (e) repeated ids, out of order, with empty slots in between: a row of
    # sel is a set (the oracle's membership test), each unit attended once
    for label, t0, L in (("repeated_chunk", w.n_ctx - 64, 64), ("repeated_single", w.n_ctx - 1, 1)):
        e = orc.num_eligible(t0 + L - 1, U, w.block, w.n_init, w.window)
        a, b_, c_ = 0, e // 2, e - 1
        row = np.array([c_, a, c_, -1, a, b_, b_, -1], np.int32)
        cases.append((label, cfg_of(w, top_k=8),
                      np.broadcast_to(row, (w.batch, w.n_kv_heads, 1, 8)).copy(), t0, L))
    _, repr_o, _ = oracle_build(orc, w, inp)
    for label, cfg, sel, t0, L in cases:
        if sel is None:
            sel = _oracle_selection(orc, w, inp, t0, L, repr_o)[:, :, None, :]
        sel_t = torch.from_numpy(np.ascontiguousarray(sel)).cuda() if sel.shape[-1] > 0 else None
        out, lse = gpu_attend(cfg, dev["q"], t0, t0, L, 1, dev["k"], dev["v"], sel_t)
        torch.cuda.synchronize()
        s0 = sel[:, :, 0] if sel.shape[-1] > 0 else np.zeros((w.batch, w.n_kv_heads, 0), np.int32)
        o_ref, l_ref = orc.attend_all(inp["q"][:, :, t0:t0 + L], t0, inp["k"], inp["v"], s0,
                                      B=w.block, n_init=w.n_init, W=w.window)
        tol = tolerance(inp["q"].dtype, o_ref)
        assert_close(out, o_ref, tol, "%s %s out" % (name, label))
        assert_close(lse, l_ref, 1e-3, "%s %s lse" % (name, label))


def test_empty_unit_pool(orc):
    """A context shorter than one unit: no units, nothing eligible, sel all -1."""
    w = CASES["bf16_g4"].replace(n_ctx=200)
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    q, k = inp["q"].cuda(), inp["k"].cuda()
    rep_idx, repr_ = gpu_build(cfg, q, k, w.n_ctx)
    assert repr_.shape[2] == 0
    scores = gpu_score(cfg, q, 100, 100, 100, 1, repr_)
    sel = gpu_topk(cfg, scores)
    torch.cuda.synchronize()
    assert (sel.cpu() == -1).all()


def test_decode_steps_parity(orc):
    """Decode: per step score(L=1) -> top-k -> attend, against the oracle."""
    w = synth.WORKLOADS["llama3_8b_128k_decode"].replace(n_ctx=6144, batch=2, n_q_heads=8,
                                                         n_kv_heads=2, decode_steps=6, top_k=8,
                                                         window=1024)
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    _, repr_g = gpu_build(cfg, dev["q"], dev["k"], w.n_ctx)
    repr_np = repr_g.cpu().double().numpy()
    U = repr_np.shape[2]
    G = w.group
    for s in range(w.decode_steps):
        t = w.n_ctx + s
        scores = gpu_score(cfg, dev["q_dec"], s, t, 1, 1, repr_g)
        sel = gpu_topk(cfg, scores)
        out, lse = gpu_attend(cfg, dev["q_dec"], s, t, 1, 1, dev["k"], dev["v"], sel)
        torch.cuda.synchronize()
        e = orc.num_eligible(t, U, w.block, w.n_init, w.window)
        sg = sel.cpu().numpy()
        for bi in range(w.batch):
            for h in range(w.n_kv_heads):
                so = orc.score_units(inp["q_dec"][bi, h * G:(h + 1) * G, s:s + 1], repr_np[bi, h], e)
                check_selection(sg[bi, h, 0], orc.topk(so, e, w.top_k), so)
        o_ref, l_ref = orc.attend_all(inp["q_dec"][:, :, s:s + 1], t, inp["k"], inp["v"],
                                      sg[:, :, 0], B=w.block, n_init=w.n_init, W=w.window)
        assert_close(out, o_ref, tolerance(torch.bfloat16, o_ref), "decode step %d" % s)
        assert_close(lse, l_ref, 1e-3, "decode lse step %d" % s)


def test_tiny_workload_pipeline(orc):
    """The tiny fp32 workload end to end (4,096 tokens, 16 chunks of 256,
    calls issued one chunk at a time), stage by stage, plus planted-unit
    recall equal to the oracle's."""
    w = synth.WORKLOADS["tiny_f32"]
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "planted_units"}
    rep_g, repr_g = gpu_build(cfg, dev["q"], dev["k"], w.n_ctx)
    torch.cuda.synchronize()
    rep_o, repr_o, ks_o = oracle_build(orc, w, inp)
    check_rep_idx(rep_g.cpu().numpy(), rep_o, ks_o, w.block, w.n_init)
    repr_np = repr_g.cpu().double().numpy()
    U = repr_np.shape[2]
    pu = w.planted_block - w.n_init // w.block
    hits_g = hits_o = n_elig = 0
    for c in range(w.n_ctx // w.chunk):
        t0 = c * w.chunk
        scores = gpu_score(cfg, dev["q"], t0, t0, w.chunk, 1, repr_g)
        sel = gpu_topk(cfg, scores)
        out, lse = gpu_attend(cfg, dev["q"], t0, t0, w.chunk, 1, dev["k"], dev["v"], sel)
        torch.cuda.synchronize()
        e = orc.num_eligible(t0 + w.chunk - 1, U, w.block, w.n_init, w.window)
        so = orc.score_units(inp["q"][0, :, t0:t0 + w.chunk], repr_np[0, 0], e)
        so_sel = orc.topk(so, e, w.top_k)
        sg = sel.cpu().numpy()[0, 0, 0]
        check_selection(sg, so_sel, so)
        if e > pu:
            n_elig += 1
            hits_g += pu in sg.tolist()
            hits_o += pu in so_sel.tolist()
        o_ref, l_ref = orc.attend_all(inp["q"][:, :, t0:t0 + w.chunk], t0, inp["k"], inp["v"],
                                      sel.cpu().numpy()[:, :, 0], B=w.block, n_init=w.n_init,
                                      W=w.window)
        assert_close(out, o_ref, 1e-4, "tiny chunk %d" % c)
        assert_close(lse, l_ref, 1e-4, "tiny lse chunk %d" % c)
    assert n_elig == 10 and hits_g == hits_o


PREFILL_VARIANTS = [
    # (G, n_init, W, chunk, n_ctx, top_k, KV heads)
    (1, 128, 512, 256, 2048, 4, 2),
    (2, 100, 200, 100, 1900, 3, 2),
    (8, 0, 64, 512, 2560, 6, 2),
    (4, 200, 300, 16, 1600, 2, 2),
    (4, 64, 4096, 512, 3072, 8, 2),    # window longer than the context: dense
    # 8 (sequence, KV head) groups: the splits of a work item share an XCD
    (2, 128, 384, 192, 1536, 4, 8),
]


@pytest.mark.parametrize("G,n_init,W,chunk,n_ctx,top_k,Hkv", PREFILL_VARIANTS)
@pytest.mark.parametrize("per_call", ["all", "one"])
def test_prefill_mfma_variants(orc, G, n_init, W, chunk, n_ctx, top_k, Hkv, per_call):
    """All chunks in one call, or one chunk per call (few workgroups: the
    tile lists are split over workgroups and merged in the kernel)."""
    w = LL.replace(n_ctx=n_ctx, n_q_heads=Hkv * G, n_kv_heads=Hkv, window=W, n_init=n_init,
                   top_k=top_k, chunk=chunk, seed=G * 1000 + n_init + Hkv)
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    _, repr_o, _ = oracle_build(orc, w, inp)
    n_chunks = n_ctx // chunk
    sels = np.stack([_oracle_selection(orc, w, inp, c * chunk, chunk, repr_o)
                     for c in range(n_chunks)], axis=2)
    checked = sorted({0, 1, n_chunks // 2, n_chunks - 1})
    sel_g = torch.from_numpy(sels).cuda()
    if per_call == "all":
        out, lse = gpu_attend(cfg, dev["q"], 0, 0, chunk, n_chunks, dev["k"], dev["v"], sel_g)
    else:
        out = torch.zeros((w.batch, w.n_q_heads, n_ctx, w.head_dim), dtype=torch.bfloat16,
                          device="cuda")
        lse = torch.zeros((w.batch, w.n_q_heads, n_ctx), dtype=torch.float32, device="cuda")
        for c in checked:
            t0 = c * chunk
            oc, lc = gpu_attend(cfg, dev["q"], t0, t0, chunk, 1, dev["k"], dev["v"],
                                sel_g[:, :, c:c + 1].contiguous())
            out[:, :, t0:t0 + chunk] = oc[:, :, :chunk]
            lse[:, :, t0:t0 + chunk] = lc[:, :, :chunk]
    torch.cuda.synchronize()
    for c in checked:
        t0 = c * chunk
        o_ref, l_ref = orc.attend_all(inp["q"][:, :, t0:t0 + chunk], t0, inp["k"], inp["v"],
                                      sels[:, :, c], B=w.block, n_init=n_init, W=W)
        assert_close(out[:, :, t0:t0 + chunk], o_ref, tolerance(torch.bfloat16, o_ref),
                     "G%d chunk %d out" % (G, c))
        assert_close(lse[:, :, t0:t0 + chunk], l_ref, 1e-3, "G%d chunk %d lse" % (G, c))


def test_prefill_deterministic_and_sequential_equals_batched(orc):
    """Two runs are bitwise equal, and one chunk per call equals all chunks
    in one call (same kernels, same reduction order)."""
    w = CASES["bf16_g4"]
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    _, repr_g = gpu_build(cfg, dev["q"], dev["k"], w.n_ctx)
    n_chunks = w.n_ctx // w.chunk
    scores = gpu_score(cfg, dev["q"], 0, 0, w.chunk, n_chunks, repr_g)
    sel = gpu_topk(cfg, scores)
    o1, l1 = gpu_attend(cfg, dev["q"], 0, 0, w.chunk, n_chunks, dev["k"], dev["v"], sel)
    o2, l2 = gpu_attend(cfg, dev["q"], 0, 0, w.chunk, n_chunks, dev["k"], dev["v"], sel)
    torch.cuda.synchronize()
    diff = (o1.float() - o2.float()).abs().max().item()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), diff
    # split-K counters are back at zero after a call on a shared workspace
    ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, w.batch, 0, w.chunk, n_chunks)
    out = torch.empty_like(o1)
    for _ in range(3):
        F.infllm_attend(cfg, dev["q"], 0, 0, w.chunk, n_chunks, dev["k"], dev["v"], sel, out,
                        None, 0, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, o1)
    if ws is not None:
        n_counters = -(-w.chunk // (128 // w.group)) * n_chunks * w.n_kv_heads * w.batch
        c0, c1, _ = F.infllm_workspace_layout(cfg, F.INFLLM_CALL_ATTEND, w.batch, 0, w.chunk,
                                              n_chunks)
        assert c1 - c0 >= 4 * n_counters
        assert int(ws[c0:c1].view(torch.int32).abs().sum()) == 0
    c = n_chunks - 2
    oc, lc = gpu_attend(cfg, dev["q"], c * w.chunk, c * w.chunk, w.chunk, 1, dev["k"], dev["v"],
                        sel[:, :, c:c + 1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(oc, o1[:, :, c * w.chunk:(c + 1) * w.chunk])


@pytest.mark.parametrize("U_big", [False, True])
def test_score_shared_workspace_repeatable(U_big):
    """Long-chunk scoring on one shared workspace: repeated calls give
    bitwise-equal scores and leave the arrival counters at zero.  U_big
    takes the two-launch path (more units than one workgroup scores)."""
    w = CASES["bf16_g4"]
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    q = inp["q"].cuda()
    U = 2600 if U_big else 24
    gen = torch.Generator().manual_seed(7)
    repr_ = torch.randn((w.batch, w.n_kv_heads, U, w.head_dim), generator=gen).cuda()
    n_chunks = 4
    ws = F.workspace(cfg, F.INFLLM_CALL_SCORE, w.batch, 0, w.chunk, n_chunks)
    outs = []
    for _ in range(3):
        sc = torch.empty((w.batch, w.n_kv_heads, n_chunks, U), dtype=torch.float32, device="cuda")
        F.infllm_score_units(cfg, q, 0, 10 ** 6, w.chunk, n_chunks, repr_, sc, ws)
        outs.append(sc)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    n_prob = w.batch * w.n_kv_heads * n_chunks
    c0, c1, _ = F.infllm_workspace_layout(cfg, F.INFLLM_CALL_SCORE, w.batch, 0, w.chunk, n_chunks)
    assert c1 - c0 >= 4 * n_prob
    assert int(ws[c0:c1].view(torch.int32).abs().sum().item()) == 0
    # against a float64 evaluation of the definition
    qs = inp["q"].double().view(w.batch, w.n_kv_heads, w.group, -1, w.head_dim)
    for c in range(n_chunks):
        qsum = qs[:, :, :, c * w.chunk:(c + 1) * w.chunk].sum(dim=(2, 3))
        ref = torch.einsum("bhd,bhud->bhu", qsum, repr_.double().cpu())
        got = outs[0][:, :, c].double().cpu()
        fin = torch.isfinite(got)
        assert torch.allclose(got[fin], ref[fin].float().double(), rtol=1e-6, atol=1e-6)


def _varlen_check(orc, w, inp, dev, cfg, repr_g, q_name, q_off, pos_list, L, n_chunks, n_oracle):
    """Score, top-k and attend with one position per sequence: each row bit
    for bit equal to the single-position call at that sequence's position
    on the same batch, and the attention against the oracle."""
    b = w.batch
    pos = torch.tensor(pos_list, dtype=torch.int64, device="cuda")
    U = repr_g.shape[2]
    q = dev[q_name]
    scores = torch.empty((b, w.n_kv_heads, n_chunks, U), dtype=torch.float32, device="cuda")
    sws = F.workspace(cfg, F.INFLLM_CALL_SCORE, b, 0, L, n_chunks)
    F.infllm_score_units_varlen(cfg, q, q_off, pos, L, n_chunks, repr_g, scores, sws)
    sel = gpu_topk(cfg, scores)
    n = L * n_chunks
    out = torch.empty((b, w.n_q_heads, n, w.head_dim), dtype=q.dtype, device="cuda")
    lse = torch.empty((b, w.n_q_heads, n), dtype=torch.float32, device="cuda")
    aws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, L, n_chunks)
    F.infllm_attend_varlen(cfg, q, q_off, pos, L, n_chunks, dev["k"], dev["v"], sel, out, lse, 0,
                           aws)
    torch.cuda.synchronize()
    sg = sel.cpu().numpy()
    for bi, t0 in enumerate(pos_list):
        s1 = gpu_score(cfg, q, q_off, t0, L, n_chunks, repr_g)
        o1, l1 = gpu_attend(cfg, q, q_off, t0, L, n_chunks, dev["k"], dev["v"], sel)
        torch.cuda.synchronize()
        assert torch.equal(scores[bi], s1[bi])
        assert torch.equal(out[bi], o1[bi]) and torch.equal(lse[bi], l1[bi])
        for c in range(n_chunks):
            e = orc.num_eligible(t0 + (c + 1) * L - 1, U, w.block, w.n_init, w.window)
            assert int(torch.isfinite(scores[bi, :, c]).sum(-1).min()) == e
        # the oracle on sampled rows of this sequence (first and last of each chunk)
        rows = sorted({c * L + r for c in range(n_chunks) for r in (0, L - 1)})[:n_oracle]
        for r in rows:
            c = r // L
            o_ref, l_ref = orc.attend_all(inp[q_name][bi:bi + 1, :, q_off + r:q_off + r + 1],
                                          t0 + r, inp["k"][bi:bi + 1], inp["v"][bi:bi + 1],
                                          sg[bi:bi + 1, :, c], B=w.block, n_init=w.n_init,
                                          W=w.window)
            assert_close(out[bi:bi + 1, :, r:r + 1], o_ref, tolerance(q.dtype, o_ref),
                         "sequence %d row %d" % (bi, r))
            assert_close(lse[bi:bi + 1, :, r:r + 1], l_ref, 1e-3, "lse sequence %d row %d" % (bi, r))
    return pos, sel, out, lse, aws


def _nan_rows_and_rest(cfg, w, dev, q_name, q_off, pos_list, L, n_chunks, sel, bad, aws):
    """A varlen attend where the sequences in `bad` have positions that do not
    fit the KV buffer: NaN rows there, the others equal to the
    single-position call, and the shared workspace still valid afterwards."""
    b = w.batch
    q = dev[q_name]
    pos = torch.tensor(pos_list, dtype=torch.int64, device="cuda")
    n = L * n_chunks
    out = torch.empty((b, w.n_q_heads, n, w.head_dim), dtype=q.dtype, device="cuda")
    lse = torch.empty((b, w.n_q_heads, n), dtype=torch.float32, device="cuda")
    F.infllm_attend_varlen(cfg, q, q_off, pos, L, n_chunks, dev["k"], dev["v"], sel, out, lse, 0,
                           aws)
    torch.cuda.synchronize()
    for bi, t0 in enumerate(pos_list):
        if bi in bad:
            assert torch.isnan(out[bi].float()).all() and torch.isnan(lse[bi]).all()
            continue
        o1, l1 = gpu_attend(cfg, q, q_off, t0, L, n_chunks, dev["k"], dev["v"], sel)
        torch.cuda.synchronize()
        assert torch.equal(out[bi], o1[bi]) and torch.equal(lse[bi], l1[bi])


def test_varlen_decode_batch(orc):
    """One decode step for four sequences at different positions (full
    context, mid context, before any unit is eligible, ragged), then with
    two positions that do not fit the KV buffer, then valid again on the
    same workspace."""
    w = synth.WORKLOADS["llama3_8b_128k_decode"].replace(n_ctx=6144, batch=4, n_q_heads=8,
                                                         n_kv_heads=2, decode_steps=4, top_k=8,
                                                         window=1024)
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    _, repr_g = gpu_build(cfg, dev["q"], dev["k"], w.n_ctx)
    cap = w.n_ctx + w.decode_steps
    pos_list = [cap - 1, 2000, 700, 4501]
    pos, sel, out, lse, aws = _varlen_check(orc, w, inp, dev, cfg, repr_g, "q_dec", 1, pos_list,
                                            1, 1, 1)
    _nan_rows_and_rest(cfg, w, dev, "q_dec", 1, [cap - 1, -1, cap, 4501], 1, 1, sel, {1, 2}, aws)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    F.infllm_attend_varlen(cfg, dev["q_dec"], 1, pos, 1, 1, dev["k"], dev["v"], sel, out2, lse2, 0,
                           aws)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


def test_varlen_chunked_prefill(orc):
    """Two 128-query chunks per sequence at different positions (MFMA
    path): a serving batch where each sequence prefills at its own offset,
    including the last position that fits the KV buffer; then one position
    past it."""
    w = CASES["bf16_g4"].replace(batch=3)
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "planted_units"}
    _, repr_g = gpu_build(cfg, dev["q"], dev["k"], w.n_ctx)
    L, nc = 128, 2
    last = w.n_ctx - L * nc
    pos_list = [last, 1000, 0]
    _, sel, _, _, aws = _varlen_check(orc, w, inp, dev, cfg, repr_g, "q", 64, pos_list, L, nc, 4)
    _nan_rows_and_rest(cfg, w, dev, "q", 64, [last + 1, 1000, 0], L, nc, sel, {0}, aws)


@pytest.mark.parametrize("U,k_m,L,nc,dup,varlen", [
    (1023, 32, 1, 1, 0, False),       # 128K decode shape
    (8191, 32, 1, 1, 0, False),       # 1M decode shape
    (1023, 32, 1, 1, 7, False),       # exact ties: repeated unit rows
    (2500, 16, 1, 2, 0, True),        # 10 keys per lane, two chunks, a position per sequence
    (9000, 8, 1, 1, 5, False),        # keys re-read from memory
    (3, 32, 1, 1, 0, False),          # fewer units than k_m
    (0, 4, 1, 1, 0, False),           # no units: all -1
    (1500, 16, 512, 2, 0, False),     # long chunks, one scoring launch + top-k launch
    (3000, 16, 512, 2, 3, True),      # long chunks beyond the one-launch limit, fused
])
def test_select_units_fused(orc, U, k_m, L, nc, dup, varlen):
    """infllm_select_units: scores bit-identical to infllm_score_units and
    selections identical to infllm_topk_units on them (and to the oracle's
    top-k on the same values), twice in a row on one workspace."""
    b, Hq, Hkv, d = 2, 8, 2, 128
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=128, n_init=128,
                        window=512, rep_k=4, top_k=k_m)
    gen = torch.Generator().manual_seed(U + 7 * k_m + L)
    q = (torch.randn((b, Hq, L * nc + 3, d), generator=gen) * 0.1).to(torch.bfloat16).cuda()
    repr_ = torch.randn((b, Hkv, max(U, 1), d), generator=gen)[:, :, :U].contiguous()
    if dup:
        repr_ = repr_[:, :, torch.arange(U) % dup].contiguous()
    repr_ = repr_.cuda()
    t_last = 128 * (U + 1) + 512 + 77        # every unit eligible at the last chunk
    pos = None
    if varlen:
        pos = torch.tensor([t_last - L * nc, 128 * (U // 2) + 512], dtype=torch.int64).cuda()
    q_pos = t_last - L * nc
    scores = torch.empty((b, Hkv, nc, U), dtype=torch.float32, device="cuda")
    sel = torch.empty((b, Hkv, nc, k_m), dtype=torch.int32, device="cuda")
    ws = F.workspace(cfg, F.INFLLM_CALL_SELECT, b, 0, L, nc)
    F.infllm_select_units(cfg, q, 3, q_pos, L, nc, repr_, scores, sel, pos=pos, ws=ws)
    # reference: the two separate calls
    ref_s = torch.empty_like(scores)
    sws = F.workspace(cfg, F.INFLLM_CALL_SCORE, b, 0, L, nc)
    if pos is None:
        F.infllm_score_units(cfg, q, 3, q_pos, L, nc, repr_, ref_s, sws)
    else:
        F.infllm_score_units_varlen(cfg, q, 3, pos, L, nc, repr_, ref_s, sws)
    ref_sel = gpu_topk(cfg, ref_s)
    sel2 = torch.full_like(sel, -5)
    F.infllm_select_units(cfg, q, 3, q_pos, L, nc, repr_, scores, sel2, pos=pos, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(scores, ref_s)
    assert torch.equal(sel, ref_sel) and torch.equal(sel2, sel)
    sg, selg = scores.cpu().double().numpy(), sel.cpu().numpy()
    for idx in np.ndindex(sg.shape[:3]):
        e = int(np.isfinite(sg[idx]).sum())
        assert selg[idx].tolist() == orc.topk(sg[idx], e, k_m).tolist()


@pytest.mark.parametrize("name", list(CASES))
def test_build_qsum_and_block_scores(orc, data, name):
    """infllm_build_units_qsum: the representations of infllm_build_units (up
    to near ties of the fp64 key scores) and block query sums equal to fp64
    sums of the queries; infllm_score_units_qsum: the scores of
    infllm_score_units for chunks of whole blocks, at an aligned offset."""
    w, inp, dev = data(name)
    cfg = cfg_of(w)
    b, Hkv, G, B, d = w.batch, w.n_kv_heads, w.group, w.block, w.head_dim
    U = F.infllm_num_units(cfg, w.n_ctx)
    nb = (w.n_ctx + B - 1) // B
    repr_ = torch.empty((b, Hkv, U, d), dtype=torch.float32, device="cuda")
    rep = (torch.empty((b, Hkv, U, w.rep_k), dtype=torch.int32, device="cuda")
           if w.rep_mode == "tokens" else None)
    bq = torch.empty((b, Hkv, nb, d), dtype=torch.float64, device="cuda")
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_QSUM, b, w.n_ctx)
    F.infllm_build_units_qsum(cfg, dev["q"], dev["k"], w.n_ctx, rep, repr_, bq, ws)
    torch.cuda.synchronize()
    # block sums against fp64 sums of the queries
    q64 = inp["q"][:, :, :w.n_ctx].double().reshape(b, Hkv, G, w.n_ctx, d).sum(2)
    want = torch.zeros((b, Hkv, nb, d), dtype=torch.float64)
    for j in range(nb):
        want[:, :, j] = q64[:, :, j * B:min((j + 1) * B, w.n_ctx)].sum(2)
    np.testing.assert_allclose(bq.cpu().numpy(), want.numpy(), rtol=1e-12, atol=1e-12)
    # representations against the oracle
    rep_o, repr_o, ks_o = oracle_build(orc, w, inp)
    rg = repr_.cpu().numpy()
    if w.rep_mode == "mean":
        np.testing.assert_array_equal(rg, repr_o.astype(np.float32))
    else:
        ex = check_rep_idx(rep.cpu().numpy(), rep_o, ks_o, B, w.n_init)
        assert len(ex) <= max(2, rep_o.shape[2] // 50)
    # chunk scores from the block sums against the ones from the queries
    L = 2 * B
    q_pos = B
    nc = (w.n_ctx - q_pos) // L
    s_blk = torch.empty((b, Hkv, nc, U), dtype=torch.float32, device="cuda")
    F.infllm_score_units_qsum(cfg, bq, q_pos, L, nc, repr_, s_blk)
    s_q = gpu_score(cfg, dev["q"], q_pos, q_pos, L, nc, repr_)
    torch.cuda.synchronize()
    a, c = s_blk.cpu().numpy(), s_q.cpu().numpy()
    assert (np.isfinite(a) == np.isfinite(c)).all()
    fin = np.isfinite(c)
    np.testing.assert_allclose(a[fin], c[fin], rtol=1e-6, atol=1e-6 * np.abs(c[fin]).max(initial=1.0))
