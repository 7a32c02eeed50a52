"""Pins for the fp64 oracle, against things other than the oracle itself:
numbers the pages print (tests/golden/pages_numbers.json), closed forms,
special cases that reduce to a library routine (torch SDPA in fp64, numpy
sorts), impulse responses and invariants.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from block_level_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


@pytest.fixture(scope="module")
def pages():
    with open(GOLDEN) as f:
        return json.load(f)


def rnd(shape, seed, dtype=torch.float32, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def sdpa64(q, k, v, mask):
    """Library attention in fp64: q [G,L,d], k/v [n,d], mask [L,n] bool."""
    q64, k64, v64 = q.double(), k.double(), v.double()
    out = torch.nn.functional.scaled_dot_product_attention(
        q64.unsqueeze(0), k64.expand(q.shape[0], -1, -1).unsqueeze(0),
        v64.expand(q.shape[0], -1, -1).unsqueeze(0), attn_mask=mask)
    logits = (q64 @ k64.T) / math.sqrt(q.shape[-1])
    lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
    return out[0].numpy(), lse.numpy()


# ------------------------------------------------------------------ unit table
def test_unit_counts_match_workload_text(orc, pages):
    for n, B, n_init, U in pages["unit_counts"]["cases"]:
        assert orc.num_units(n, B, n_init) == U


def test_unit_figure_alignment(orc, pages):
    f = pages["unit_figure"]
    B = f["B"]
    # with any sink count below the figure's first token, some unit spans
    # exactly tokens 1024..1151
    for n_init in (4, 64, 128, 1000):
        spans = [orc.unit_keys(u, B, n_init) for u in range(orc.num_units(4096, B, n_init))]
        assert (f["first_token"], f["last_token"] + 1) in spans


def test_units_at_one_million(orc, pages):
    f = pages["units_at_1m"]
    for n_init in (4, 16, 128):
        U = orc.num_units(f["n_tokens"], f["B"], n_init)
        assert abs(U - f["approx_units"]) <= f["rel_tol"] * f["approx_units"]


def test_partial_first_unit_excludes_sinks(orc):
    assert orc.unit_keys(0, 128, 64) == (64, 128)
    assert orc.unit_keys(0, 128, 128) == (128, 256)
    assert orc.unit_keys(3, 32, 40) == (128, 160)
    assert orc.num_units(4096, 128, 64) == 32
    assert orc.num_units(100, 128, 0) == 0


def test_eligible_prefix_closed_form(orc):
    # n_init a multiple of B: e = clamp(floor((t_last - W)/B) - n_init/B + 1, 0, U)
    for B, n_init, W, n in [(128, 128, 4096, 32768), (32, 64, 96, 1024), (16, 0, 16, 400)]:
        U = orc.num_units(n, B, n_init)
        for t_last in range(0, n, 7):
            x = t_last - W
            want = 0 if x < n_init else min(U, x // B - n_init // B + 1)
            assert orc.num_eligible(t_last, U, B, n_init, W) == want, (B, n_init, W, t_last)


# ---------------------------------------------------------- working context
def test_n_active_matches_pages(orc, pages):
    f = pages["n_active"]
    B, n_init, W = f["L_unit"], f["T_sink"], f["W_local"]
    t = 50_000
    sel = [40, 41, 100, 200]            # four full units far behind the window
    assert orc.working_context(t, sel, B, n_init, W).size == f["N_active"]


def test_streaming_active_matches_pages(orc, pages):
    f = pages["streaming_active"]
    t = 70_000
    n = orc.working_context(t, [], 128, f["T_sink"], f["W_local"]).size
    assert n == f["T_sink"] + f["W_local"]
    assert int(n * f["bytes_per_token"] / 1e6) == f["mb_printed"]


def test_chunk_bound(orc, pages):
    f = pages["chunk_bound"]
    B, n_init, W, k_m, C = f["B"], f["n_init"], f["W"], f["k_m"], f["chunk"]
    sel = list(range(0, 16 * 3, 3))
    sizes = [orc.working_context(t, sel, B, n_init, W).size for t in range(20 * C, 21 * C)]
    assert max(sizes) == f["bound"]
    # a selected unit straddling t - W contributes only its keys <= t - W
    t = 20 * C
    j = (t - W) // B
    part = orc.working_context(t, [j - n_init // B], B, n_init, W)
    assert part.size == n_init + W + ((t - W) - j * B + 1)


def test_working_context_definition_small(orc):
    B, n_init, W = 4, 3, 5
    sel = [1, 4]                        # blocks 1 and 4 -> keys 4..7, 16..19
    t = 30
    want = [0, 1, 2, 4, 5, 6, 7, 16, 17, 18, 19] + list(range(26, 31))
    assert orc.working_context(t, sel, B, n_init, W).tolist() == want
    # early query: causal, sinks and window overlap
    assert orc.working_context(2, sel, B, n_init, W).tolist() == [0, 1, 2]
    assert orc.working_context(9, [0, 1], B, n_init, W).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 8, 9]
    # the membership predicate itself: nothing after the query, in any part
    for p in (0, 2, 5, 16, 29, 30):
        assert orc.in_working_context(p, t, sel, B, n_init, W)
        assert not orc.in_working_context(t + 1 + p, t, sel, B, n_init, W)
    assert not orc.in_working_context(3, 30, sel, B, n_init, W)


# -------------------------------------------------------- representative scores
def test_rep_score_impulse_response(orc):
    G, n, d, W = 3, 200, 8, 17
    qg = torch.zeros(G, n, d)
    istar = 120
    qg[:, istar] = rnd((G, d), 1)
    k = rnd((n, d), 2)
    want = (qg[:, istar].double().sum(0) @ k.double().T).numpy()
    for p in range(n):
        s = orc.rep_score(qg, k, n, W, p)
        if istar - W <= p <= istar - 1:
            assert s == pytest.approx(want[p], rel=1e-12, abs=1e-12)
        else:
            assert s == 0.0


def test_rep_score_constant_queries(orc):
    G, n, d, W = 2, 300, 4, 40
    e = torch.tensor([0.5, -1.0, 2.0, 0.25])
    qg = e.expand(G, n, d).contiguous()
    k = rnd((n, d), 3)
    for p in [0, 1, 100, n - W - 1, n - W, n - 10, n - 1]:
        count = min(p + W, n - 1) - p
        want = G * count * float(k[p].double() @ e.double())
        assert orc.rep_score(qg, k, n, W, p) == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_rep_score_bf16_widening_exact(orc):
    G, n, d, W = 2, 64, 16, 8
    qg = rnd((G, n, d), 4, torch.bfloat16)
    k = rnd((n, d), 5, torch.bfloat16)
    for p in (0, 30, 63):
        assert orc.rep_score(qg, k, n, W, p) == orc.rep_score(qg.float(), k.float(), n, W, p)


# ------------------------------------------------------------- representatives
def test_representatives_follow_key_ranking(orc):
    # constant queries along e0: score_p = G*count(p)*k_p[0]; away from the
    # context end count = W, so the representatives are the r_k largest k[0]
    G, d, B, n_init, W, r_k = 2, 8, 16, 16, 32, 3
    n = 256
    qg = torch.zeros(G, n, d)
    qg[:, :, 0] = 1.0
    k = rnd((n, d), 6)
    U = orc.num_units(n, B, n_init)
    rep_idx, repr_, ks = orc.build_tokens(qg, k, n, B, n_init, W, r_k)
    for u in range(U):
        lo, hi = orc.unit_keys(u, B, n_init)
        if hi + W > n:
            continue
        order = np.argsort(-k[lo:hi, 0].numpy(), kind="stable")[:r_k] + lo
        assert rep_idx[u].tolist() == sorted(order.tolist())
        np.testing.assert_allclose(repr_[u], k[sorted(order.tolist())].double().sum(0).numpy(),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(ks[u], (G * W * k[lo:hi, 0].double()).numpy(), rtol=1e-12)


def test_representative_ties_take_lower_position(orc):
    G, d, B, n_init, W, r_k = 1, 4, 8, 8, 16, 3
    n = 128
    qg = torch.ones(G, n, d)
    k = torch.ones(n, d)
    rep_idx, _, _ = orc.build_tokens(qg, k, n, B, n_init, W, r_k)
    for u in range(orc.num_units(n, B, n_init)):
        lo, hi = orc.unit_keys(u, B, n_init)
        if hi + W <= n:
            assert rep_idx[u].tolist() == [lo, lo + 1, lo + 2]


def test_all_keys_representative_equals_block_mean(orc):
    G, d, B, n_init, W = 2, 8, 16, 32, 24
    n = 320
    qg, k = rnd((G, n, d), 7), rnd((n, d), 8)
    U = orc.num_units(n, B, n_init)
    _, repr_tok, _ = orc.build_tokens(qg, k, n, B, n_init, W, B)
    repr_mean = orc.build_mean(k, B, n_init, 0, U)
    np.testing.assert_allclose(repr_tok, B * repr_mean, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(repr_mean[2], k[64:80].double().mean(0).numpy(), atol=1e-14)


def test_partial_unit_representatives(orc):
    G, d, B, n_init, W, r_k = 1, 8, 32, 20, 16, 4
    n = 160
    qg, k = rnd((G, n, d), 9), rnd((n, d), 10)
    rep_idx, _, ks = orc.build_tokens(qg, k, n, B, n_init, W, r_k)
    assert all(20 <= p < 32 for p in rep_idx[0])
    assert np.isnan(ks[0, :20]).all() and np.isfinite(ks[0, 20:]).all()
    assert orc.build_mean(k, B, n_init, 0, 1)[0] == pytest.approx(
        k[20:32].double().mean(0).numpy(), abs=1e-14)
    # fewer keys than r_k: pad with -1
    rep_idx2, _, _ = orc.build_tokens(qg, k, n, B, 30, W, r_k)
    assert sorted(rep_idx2[0].tolist()) == [-1, -1, 30, 31]


def test_streaming_build_truncation(orc):
    """A unit built at a shorter context: its key scores sum only the queries
    before that context's end (R1 with n_ctx as the current position), so a
    unit whose last key is at or before n_ctx-1-W (every key's window inside
    the context) gets exactly its whole-context result, and a unit still in
    the window differs only through the truncated sums.  Checked against
    direct sums of q.k over the truncated windows."""
    G, d, B, n_init, W, r_k = 2, 8, 32, 32, 48, 3
    n = 400
    qg, k = rnd((G, n, d), 21), rnd((n, d), 22)
    rep_f, repr_f, ks_f = orc.build_tokens(qg, k, n, B, n_init, W, r_k)
    for n_cur in (150, 211, 300):
        U = orc.num_units(n_cur, B, n_init)
        rep_c, repr_c, ks_c = orc.build_tokens(qg, k, n_cur, B, n_init, W, r_k, 0, U)
        for u in range(U):
            lo, hi = orc.unit_keys(u, B, n_init)
            # key scores: direct sums over p+1 .. min(p+W, n_cur-1)
            for p in range(lo, hi):
                end = min(p + W, n_cur - 1)
                want = float((qg[:, p + 1:end + 1].double().sum((0, 1)) @ k[p].double()))
                assert ks_c[u, p - (u + n_init // B) * B] == pytest.approx(want, rel=1e-12,
                                                                           abs=1e-12)
            if hi - 1 <= n_cur - 1 - W:
                assert rep_c[u].tolist() == rep_f[u].tolist()
                assert np.array_equal(repr_c[u], repr_f[u])
        # and a range call equals the same rows of the whole-range call
        lo_u = U // 2
        rep_r, repr_r, _ = orc.build_tokens(qg, k, n_cur, B, n_init, W, r_k, lo_u, U)
        assert np.array_equal(rep_r, rep_c[lo_u:]) and np.array_equal(repr_r, repr_c[lo_u:])


# --------------------------------------------------------------- unit scores
def test_chunk_score_bilinear_expansion(orc):
    G, d, B, n_init, W, r_k = 3, 8, 16, 16, 32, 2
    n, t0, L = 400, 300, 37
    qg, k = rnd((G, n, d), 11), rnd((n, d), 12)
    U = orc.num_units(n, B, n_init)
    rep_idx, repr_, _ = orc.build_tokens(qg, k, n, B, n_init, W, r_k)
    e = orc.num_eligible(t0 + L - 1, U, B, n_init, W)
    scores = orc.score_units(qg[:, t0:t0 + L], repr_, e)
    qq = qg[:, t0:t0 + L].double().reshape(-1, d).numpy()
    kk = k.double().numpy()
    for u in range(U):
        if u >= e:
            assert scores[u] == -math.inf
            continue
        want = sum(float(qq[i] @ kk[p]) for i in range(qq.shape[0]) for p in rep_idx[u])
        assert scores[u] == pytest.approx(want, rel=1e-10, abs=1e-10)


def test_chunk_score_is_sum_of_query_scores(orc):
    G, d, U = 2, 16, 10
    qg = rnd((G, 9, d), 13)
    repr_ = rnd((U, d), 14).double().numpy()
    whole = orc.score_units(qg, repr_, U)
    parts = sum(orc.score_units(qg[:, i:i + 1], repr_, U) for i in range(9))
    np.testing.assert_allclose(whole, parts, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------- top-k
def test_topk_against_lexsort(orc):
    rng = np.random.default_rng(0)
    for trial in range(50):
        U = int(rng.integers(1, 60))
        e = int(rng.integers(0, U + 1))
        k_m = int(rng.integers(1, 20))
        s = rng.integers(-5, 5, size=U).astype(np.float64)      # many ties
        s[e:] = -math.inf
        sel = orc.topk(s, e, k_m)
        order = np.lexsort((np.arange(e), -s[:e]))[:min(k_m, e)]
        want = sorted(order.tolist()) + [-1] * (k_m - min(k_m, e))
        assert sel.tolist() == want, (U, e, k_m)


def test_dominant_unit_always_retrieved(orc):
    # a unit whose keys all point along the chunk's query sum, longer than
    # any other key, has the largest score by Cauchy-Schwarz
    b, Hkv, G, d, B, n_init, W = 1, 2, 2, 16, 16, 16, 64
    n, C = 512, 32
    q = rnd((b, Hkv * G, n, d), 15)
    k = rnd((b, Hkv, n, d), 16)
    for t0 in (128, 256, 480):
        for block in (1, 3, (t0 + C - 1 - W) // B):
            kk = k.clone()
            qsum = q[:, :, t0:t0 + C].double().sum(2).reshape(b, Hkv, G, d).sum(2)
            synth.plant_dominant_block(kk, block, B, qsum)
            for mode in ("tokens", "mean"):
                _, repr_, _ = orc.build_units_all(q, kk, n, B=B, n_init=n_init, W=W, r_k=2,
                                                  mode=mode)
                _, sel, e = orc.select_all(q[:, :, t0:t0 + C], t0, repr_, B=B, n_init=n_init,
                                           W=W, k_m=1)
                assert (sel[0, :, 0] == block - n_init // B).all(), (t0, block, mode)


def test_ineligible_unit_never_selected(orc):
    b, Hkv, G, d, B, n_init, W = 1, 1, 2, 16, 16, 16, 64
    n, C, t0 = 512, 32, 400
    q, k = rnd((b, G, n, d), 17), rnd((b, Hkv, n, d), 18)
    block = (t0 + C - 1 - W) // B + 1        # first key inside the last query's window
    qsum = q[:, :, t0:t0 + C].double().sum(2).reshape(b, Hkv, G, d).sum(2)
    synth.plant_dominant_block(k, block, B, qsum)
    _, repr_, _ = orc.build_units_all(q, k, n, B=B, n_init=n_init, W=W, r_k=2)
    _, sel, e = orc.select_all(q[:, :, t0:t0 + C], t0, repr_, B=B, n_init=n_init, W=W, k_m=3)
    assert e == block - n_init // B
    assert (block - n_init // B) not in sel[0, 0].tolist()


# ----------------------------------------------------------------- attention
def _mask(t0, L, n, fn):
    return torch.tensor([[fn(t0 + i, p) for p in range(n)] for i in range(L)])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_all_units_selected_equals_dense_causal(orc, dtype):
    G, d, B, n_init, W = 2, 16, 16, 8, 48
    n = 400
    q, k, v = rnd((G, n, d), 19, dtype), rnd((n, d), 20, dtype), rnd((n, d), 21, dtype)
    U = orc.num_units(n, B, n_init)
    for t0, L in [(0, 64), (100, 50), (350, 50), (399, 1)]:
        sel = list(range(U))                    # k_m >= eligible: every unit
        out, lse = orc.attend(q[:, t0:t0 + L], t0, k, v, sel, B, n_init, W)
        m = _mask(t0, L, n, lambda t, p: p <= t)
        want, want_lse = sdpa64(q[:, t0:t0 + L], k, v, m)
        np.testing.assert_allclose(out, want, atol=1e-12)
        np.testing.assert_allclose(lse, want_lse, atol=1e-12)


def test_no_units_is_sinks_plus_window(orc):
    G, d, B, n_init, W = 2, 16, 16, 5, 37
    n = 300
    q, k, v = rnd((G, n, d), 22), rnd((n, d), 23), rnd((n, d), 24)
    t0, L = 200, 60
    out, lse = orc.attend(q[:, t0:t0 + L], t0, k, v, [-1, -1], B, n_init, W)
    m = _mask(t0, L, n, lambda t, p: p <= t and (p < n_init or p > t - W))
    want, want_lse = sdpa64(q[:, t0:t0 + L], k, v, m)
    np.testing.assert_allclose(out, want, atol=1e-12)
    np.testing.assert_allclose(lse, want_lse, atol=1e-12)


def test_window_covering_context_is_dense(orc):
    G, d, B, n_init, W = 1, 8, 16, 4, 1000
    n = 200
    q, k, v = rnd((G, n, d), 25), rnd((n, d), 26), rnd((n, d), 27)
    out, _ = orc.attend(q, 0, k, v, [-1], B, n_init, W)
    want, _ = sdpa64(q, k, v, _mask(0, n, n, lambda t, p: p <= t))
    np.testing.assert_allclose(out, want, atol=1e-12)


def test_selected_units_match_explicit_mask(orc):
    G, d, B, n_init, W = 2, 8, 8, 8, 24
    n = 256
    q, k, v = rnd((G, n, d), 28), rnd((n, d), 29), rnd((n, d), 30)
    sel = [2, 9, 20]
    blocks = {u + n_init // B for u in sel}
    t0, L = 180, 40
    out, _ = orc.attend(q[:, t0:t0 + L], t0, k, v, sel, B, n_init, W)
    m = _mask(t0, L, n, lambda t, p: p <= t and (
        p < n_init or p > t - W or (p // B in blocks and p <= t - W)))
    want, _ = sdpa64(q[:, t0:t0 + L], k, v, m)
    np.testing.assert_allclose(out, want, atol=1e-12)
    # order of sel is irrelevant
    out2, _ = orc.attend(q[:, t0:t0 + L], t0, k, v, [20, 2, 9], B, n_init, W)
    np.testing.assert_array_equal(out, out2)


def test_decode_equals_chunk_of_one(orc):
    G, d, B, n_init, W = 2, 8, 8, 8, 24
    n = 256
    q, k, v = rnd((G, n, d), 31), rnd((n, d), 32), rnd((n, d), 33)
    sel = [1, 5, 17]
    out, _ = orc.attend(q[:, 100:140], 100, k, v, sel, B, n_init, W)
    for i in (0, 17, 39):
        o1, _ = orc.attend(q[:, 100 + i:101 + i], 100 + i, k, v, sel, B, n_init, W)
        np.testing.assert_array_equal(o1[:, 0], out[:, i])


def test_two_key_closed_form(orc):
    d = 4
    q = torch.tensor([[[1.0, 2.0, 0.0, -1.0]]])
    k = torch.tensor([[0.5, 0.0, 1.0, 1.0], [1.0, 1.0, 0.0, 0.0]])
    v = torch.tensor([[1.0, 0.0, 2.0, 0.0], [0.0, 3.0, 0.0, 1.0]])
    out, lse = orc.attend(q, 1, k, v, [-1], 8, 1, 1)        # sink 0 + window {1}
    s = [(-0.5) / 2.0, 3.0 / 2.0]
    w0 = math.exp(s[0]) / (math.exp(s[0]) + math.exp(s[1]))
    np.testing.assert_allclose(out[0, 0], w0 * v[0].double().numpy() + (1 - w0) * v[1].double().numpy(),
                               atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(s[0]) + math.exp(s[1])), abs=1e-15)
