"""Pins of the oracle's in-attention positions (InfLLM Guide, "Operational
Checklist", RoPE item: native base kept, local relative offsets within
memory units).  Reading pinned here: q and k arrive rotated at their absolute
positions; the attention re-indexes them to their place in the working
context (initial tokens first, then the selected units in slot order, then
the local tokens).  The references below are written independently of the
oracle: a textbook rotate-half RoPE in numpy and plain softmax attention
over an explicitly assembled cache whose positions are the cache order."""
import numpy as np
import pytest
import torch

THETA = 10000.0


def rope_np(x, pos, theta=THETA):
    """Textbook rotary embedding, rotate-half pairing: pair (c, c + d/2)
    turned by pos * theta^(-2c/d).  x [..., d]; pos broadcast to x[..., 0]."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    inv = theta ** (-2.0 * np.arange(h) / d)
    a = np.asarray(pos, np.float64)[..., None] * inv
    c, s = np.cos(a), np.sin(a)
    x0, x1 = x[..., :h], x[..., h:]
    return np.concatenate([x0 * c - x1 * s, x1 * c + x0 * s], axis=-1)


def softmax_attend(q, k, v):
    """q [d], k/v [n, d] -> out [d], lse."""
    lg = k @ q / np.sqrt(q.shape[-1])
    m = lg.max()
    w = np.exp(lg - m)
    return (w[:, None] * v).sum(0) / w.sum(), m + np.log(w.sum())


def absolute_inputs(n, d, seed):
    """Raw q/k/v and their copies rotated at absolute positions, as fp32
    arrays (the oracle reads the fp32 values; the references un-rotate the
    same fp32 values in fp64)."""
    g = np.random.default_rng(seed)
    qr = g.standard_normal((n, d))
    kr = g.standard_normal((n, d))
    v = g.standard_normal((n, d)).astype(np.float32)
    pos = np.arange(n)
    qa = rope_np(qr, pos).astype(np.float32)
    ka = rope_np(kr, pos).astype(np.float32)
    return qa, ka, v


def oracle_decode(orc, qa, ka, v, t, sel, B, n_init, W, theta=THETA):
    o, l = orc.attend(torch.from_numpy(qa[t:t + 1][None]), t, torch.from_numpy(ka),
                      torch.from_numpy(v), np.asarray(sel, np.int32), B, n_init, W, theta)
    return o[0, 0], l[0, 0]


def cache_reference(qa, ka, v, t, cache_tokens):
    """Attention of query t over the cache [cache_tokens] whose positions are
    0 .. n-1 in that order, the query at n-1 (inputs un-rotated from their
    absolute positions first)."""
    idx = np.asarray(cache_tokens)
    q = rope_np(rope_np(qa[t].astype(np.float64), -t), len(idx) - 1)
    k = rope_np(rope_np(ka[idx].astype(np.float64), -idx), np.arange(len(idx)))
    return softmax_attend(q, k, v[idx].astype(np.float64))


def test_dense_window_keeps_absolute_positions(orc):
    """No units, a window over the whole context: every position stays
    absolute, so re-indexing changes nothing."""
    d, n = 32, 300
    qa, ka, v = absolute_inputs(n, d, 1)
    for t in (0, 5, 150, 299):
        o_r, l_r = oracle_decode(orc, qa, ka, v, t, [], 64, 16, 4096)
        o_p, l_p = oracle_decode(orc, qa, ka, v, t, [], 64, 16, 4096, theta=0.0)
        np.testing.assert_allclose(o_r, o_p, atol=1e-10)
        assert abs(l_r - l_p) < 1e-10


@pytest.mark.parametrize("t", [200, 333, 700])
def test_no_units_is_streaming_cache(orc, t):
    """k_m = 0: the initial tokens and the window form the cache, positioned
    by their order in it (StreamingLLM with re-indexed positions)."""
    d, n, B, n_init, W = 32, 800, 64, 16, 100
    qa, ka, v = absolute_inputs(n, d, 2)
    cache = list(range(n_init)) + list(range(max(n_init, t - W + 1), t + 1))
    o_ref, l_ref = cache_reference(qa, ka, v, t, cache)
    o, l = oracle_decode(orc, qa, ka, v, t, [], B, n_init, W)
    np.testing.assert_allclose(o, o_ref, atol=1e-10)
    assert abs(l - l_ref) < 1e-10


@pytest.mark.parametrize("order", ["ascending", "reversed"])
def test_units_next_to_window_form_contiguous_cache(orc, order):
    """Two selected units in the blocks right before the window (which starts
    on a block boundary): the cache is initial tokens, the unit in slot 0,
    the unit in slot 1, the window -- positioned by that order, so the slot
    order (not the unit order) decides where a unit sits."""
    d, B, n_init, W = 32, 64, 64, 128
    t = 10 * B + W - 1                   # window [10B, 10B + W)
    n = t + 1
    qa, ka, v = absolute_inputs(n, d, 3)
    j_a, j_b = 8, 9                      # blocks 8 and 9 -> units 7 and 8 (n_init/B = 1)
    units = [j_a - 1, j_b - 1] if order == "ascending" else [j_b - 1, j_a - 1]
    blocks = [u + 1 for u in units]
    cache = list(range(n_init))
    for j in blocks:
        cache += list(range(j * B, (j + 1) * B))
    cache += list(range(10 * B, t + 1))
    o_ref, l_ref = cache_reference(qa, ka, v, t, cache)
    o, l = oracle_decode(orc, qa, ka, v, t, units, B, n_init, W)
    np.testing.assert_allclose(o, o_ref, atol=1e-10)
    assert abs(l - l_ref) < 1e-10


def test_positions_independent_of_absolute_offset(orc):
    """The same raw content placed a multiple of B later (initial tokens
    unchanged, selected units shifted with it): every working-context
    position is unchanged, so are the outputs, for every query of a chunk."""
    d, B, n_init, W, L, shift = 32, 64, 64, 128, 48, 5 * 64
    n = 1200
    g = np.random.default_rng(4)
    qr, kr = g.standard_normal((n + shift, d)), g.standard_normal((n + shift, d))
    vr = g.standard_normal((n + shift, d))
    # second copy: tokens >= n_init moved by `shift`
    def place(x, s):
        y = np.zeros_like(x)
        y[:n_init] = x[:n_init]
        y[n_init + s:n + s] = x[n_init:n]
        return y
    outs = []
    sel_a = np.array([3, 9, 5, -1], np.int32)
    for s in (0, shift):
        pos = np.arange(n + shift)
        qa = rope_np(place(qr, s), pos).astype(np.float32)
        ka = rope_np(place(kr, s), pos).astype(np.float32)
        v = place(vr, s).astype(np.float32)
        sel = np.where(sel_a >= 0, sel_a + s // B, -1).astype(np.int32)
        t0 = 1000 + s
        o, l = orc.attend(torch.from_numpy(qa[t0:t0 + L][None].repeat(2, 0)), t0,
                          torch.from_numpy(ka), torch.from_numpy(v), sel, B, n_init, W, THETA)
        outs.append((o, l))
    # equal up to the fp32 rounding of the two inputs (each rotated at its own
    # absolute positions before rounding)
    np.testing.assert_allclose(outs[0][0], outs[1][0], atol=1e-6)
    np.testing.assert_allclose(outs[0][1], outs[1][1], atol=1e-6)
    # and the re-indexing does matter here: not the absolute-position result
    o_abs, _ = orc.attend(torch.from_numpy(qa[t0:t0 + L][None].repeat(2, 0)), t0,
                          torch.from_numpy(ka), torch.from_numpy(v), sel, B, n_init, W, 0.0)
    assert np.abs(o_abs - outs[1][0]).max() > 1e-3


def test_context_positions_bounded(orc):
    """Every attended position of a chunk lies below n_init + k_m*B + W + L
    (the distances stay within the pretrained range whatever the context
    length), and the initial tokens keep their own positions."""
    B, n_init, W, L, k_m = 128, 128, 4096, 512, 16
    sel = np.arange(0, 2 * k_m, 2, dtype=np.int32)
    for t0 in (8192, 1 << 20):
        top = n_init + k_m * B + W + L
        for p in list(range(0, n_init, 37)) + [t0 - W + 1, t0, t0 + L - 1]:
            cp = orc.context_pos(p, t0, sel, B, n_init, W)
            assert 0 <= cp < top
        assert orc.context_pos(5, t0, sel, B, n_init, W) == 5
        # a key of the unit in slot 3 keeps its offset in the block
        u = int(sel[3])
        p = (u + n_init // B) * B + 17
        assert orc.context_pos(p, t0, sel, B, n_init, W) == n_init + 3 * B + 17
