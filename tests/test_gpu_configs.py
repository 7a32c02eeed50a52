"""GPU parity over a seeded spread of valid configurations (group sizes,
head sizes, unit sizes, sink counts, windows, k_m, dtypes, chunk lengths
including ragged last chunks, per-sequence positions), each through the
whole path -- range-built pool, fused selection, attention -- against the
oracle stage by stage on the GPU's upstream outputs."""
import numpy as np
import pytest
import torch

from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth
from gpu_helpers import assert_close, cfg_of, check_rep_idx, check_selection, tolerance

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    B = int(rng.choice([64, 128]))
    n_init = int(rng.choice([0, 17, 64, 130]))
    W = int(rng.choice([100, 256, 513]))
    top_k = int(rng.choice([1, 3, 8, 20]))
    rep_mode = str(rng.choice(["tokens", "mean"]))
    n_ctx = int(rng.integers(n_init + W + 4 * B, n_init + W + 16 * B))
    L = int(rng.choice([1, 16, 100, 256]))
    n_chunks = int(rng.integers(1, 4))
    w = synth.WORKLOADS["tiny_f32"].replace(
        batch=2, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=d, dtype=dtype, block=B,
        n_init=n_init, window=W, rep_k=int(rng.integers(1, 5)), top_k=top_k, rep_mode=rep_mode,
        n_ctx=n_ctx, chunk=L, decode_steps=0, planted="none", seed=1000 + seed,
        scale=1.0 if dtype == "f32" else 0.09)
    return w, L, n_chunks, rng


@pytest.mark.parametrize("seed", range(40))
def test_random_config(orc, seed):
    w, L, nc, rng = draw(seed)
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    b, Hkv, G, B = w.batch, w.n_kv_heads, w.group, w.block
    # the pool: two range calls (start, then the rest) at the full context
    U = F.infllm_num_units(cfg, w.n_ctx)
    repr_ = torch.full((b, Hkv, U, w.head_dim), float("nan"), device="cuda")
    rep = (torch.full((b, Hkv, U, w.rep_k), -7, dtype=torch.int32, device="cuda")
           if w.rep_mode == "tokens" else None)
    cut = U // 3
    for lo, hi in ((0, cut), (cut, U)):
        ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_RANGE, b, max(hi - lo, 1))
        F.infllm_build_units_range(cfg, dev["q"], dev["k"], w.n_ctx, lo, hi, rep, repr_, ws)
    torch.cuda.synchronize()
    rep_o, repr_o, ks_o = orc.build_units_all(inp["q"], inp["k"], w.n_ctx, B=B, n_init=w.n_init,
                                             W=w.window, r_k=w.rep_k, mode=w.rep_mode)
    rg = repr_.cpu().numpy()
    if w.rep_mode == "mean":
        np.testing.assert_array_equal(rg, repr_o.astype(np.float32))
    else:
        ex = check_rep_idx(rep.cpu().numpy(), rep_o, ks_o, B, w.n_init)
        assert len(ex) <= max(2, U * b * Hkv // 50)
    # chunks at per-sequence positions (the last chunk ends at the context end)
    n = L * nc
    pos = [w.n_ctx - n, int(rng.integers(0, w.n_ctx - n + 1))]
    pos_t = torch.tensor(pos, dtype=torch.int64, device="cuda")
    q_off = int(rng.integers(0, w.n_ctx - n + 1))
    scores = torch.empty((b, Hkv, nc, U), dtype=torch.float32, device="cuda")
    sel = torch.empty((b, Hkv, nc, w.top_k), dtype=torch.int32, device="cuda")
    sws = F.workspace(cfg, F.INFLLM_CALL_SELECT, b, 0, L, nc)
    F.infllm_select_units(cfg, dev["q"], q_off, 0, L, nc, repr_, scores, sel, pos=pos_t, ws=sws)
    out = torch.empty((b, w.n_q_heads, n, w.head_dim), dtype=dev["q"].dtype, device="cuda")
    lse = torch.empty((b, w.n_q_heads, n), dtype=torch.float32, device="cuda")
    aws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, L, nc)
    F.infllm_attend_varlen(cfg, dev["q"], q_off, pos_t, L, nc, dev["k"], dev["v"], sel, out, lse,
                           0, aws)
    torch.cuda.synchronize()
    rn = repr_.cpu().double().numpy()
    sg, selg = scores.cpu().numpy(), sel.cpu().numpy()
    for bi in range(b):
        for c in range(nc):
            t_last = pos[bi] + (c + 1) * L - 1
            e = orc.num_eligible(t_last, U, B, w.n_init, w.window)
            for h in range(Hkv):
                rows = inp["q"][bi, h * G:(h + 1) * G, q_off + c * L:q_off + (c + 1) * L]
                so = orc.score_units(rows, rn[bi, h], e)
                fin = np.isfinite(so)
                assert (np.isfinite(sg[bi, h, c]) == fin).all()
                np.testing.assert_allclose(sg[bi, h, c][fin], so[fin], rtol=1e-6,
                                           atol=1e-6 * np.abs(so[fin]).max(initial=1.0))
                assert selg[bi, h, c].tolist() == orc.topk(sg[bi, h, c].astype(np.float64), e,
                                                             w.top_k).tolist()
                check_selection(selg[bi, h, c], orc.topk(so, e, w.top_k), so)
            for r in sorted({c * L, c * L + L - 1, c * L + L // 2}):
                o_ref, l_ref = orc.attend_all(inp["q"][bi:bi + 1, :, q_off + r:q_off + r + 1],
                                              pos[bi] + r, inp["k"][bi:bi + 1],
                                              inp["v"][bi:bi + 1], selg[bi:bi + 1, :, c],
                                              B=B, n_init=w.n_init, W=w.window)
                assert_close(out[bi:bi + 1, :, r:r + 1], o_ref, tolerance(dev["q"].dtype, o_ref),
                             "seed %d seq %d row %d" % (seed, bi, r))
                assert_close(lse[bi:bi + 1, :, r:r + 1], l_ref, 1e-3, "lse seed %d" % seed)
