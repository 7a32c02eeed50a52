"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (bench.Pipeline: one score/top-k/attend call covering all
chunks of the encoding pass, one per decode step).  The oracle checks what it can afford one by one:
  - the unit build on contiguous samples of units (start, middle and end of
    the context, where the representative window is truncated);
  - every chunk's and every decode step's selection, re-derived from the
    oracle's fp64 scores on the GPU's unit representations (near-tie rule);
  - attention outputs at sampled query positions / decode steps, on the
    GPU's own selections;
  - for the 1M workload, planted-unit recall equal to the oracle's.
"""
import numpy as np
import pytest
import torch

import bench
from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth
from gpu_helpers import assert_close, check_selection, tolerance

pytestmark = pytest.mark.gpu


def run(name, rope_theta=0.0, **over):
    w = synth.WORKLOADS[name]
    if over:
        w = w.replace(**over)
    p = bench.Pipeline(w, rope_theta=rope_theta)
    if not p.encode:
        p.build()
    p.step()
    torch.cuda.synchronize()
    return w, p


def check_build(orc, w, p, samples, n_ctx=None, rep_idx=None, repr_=None):
    """samples: list of (b, h, u_lo, u_hi); by default the pipeline's own
    pool, built at the workload's context."""
    G, B = w.group, w.block
    n_ctx = w.n_ctx if n_ctx is None else n_ctx
    rep_idx = p.rep_idx if rep_idx is None else rep_idx
    repr_ = p.repr if repr_ is None else repr_
    exemptions = 0
    for bi, h, u_lo, u_hi in samples:
        k = p.inp["k"][bi, h, :n_ctx].cpu()
        repr_g = repr_[bi, h, u_lo:u_hi].cpu().numpy()
        if w.rep_mode == "mean":
            repr_o = orc.build_mean(k, B, w.n_init, u_lo, u_hi)
            np.testing.assert_array_equal(repr_g, repr_o.astype(np.float32))
            continue
        qg = p.inp["q"][bi, h * G:(h + 1) * G, :n_ctx].cpu()
        rep_o, repr_o, ks_o = orc.build_tokens(qg, k, n_ctx, B, w.n_init, w.window, w.rep_k,
                                               u_lo, u_hi)
        rep_g = rep_idx[bi, h, u_lo:u_hi].cpu().numpy()
        for i in range(u_hi - u_lo):
            if np.array_equal(rep_g[i], rep_o[i]):
                np.testing.assert_array_equal(repr_g[i], repr_o[i].astype(np.float32))
                continue
            start = (u_lo + i + w.n_init // B) * B
            by_pos = {start + s: ks_o[i, s] for s in range(B) if np.isfinite(ks_o[i, s])}
            exemptions += check_selection(rep_g[i], rep_o[i], by_pos)
    assert exemptions <= max(1, sum(s[3] - s[2] for s in samples) // 20)


def check_selections(orc, w, p, q_cpu, sel_log, items):
    """items: (index into sel_log, first query row, first position, L)."""
    G = w.group
    repr_np = p.repr.cpu().double().numpy()
    sel = sel_log.cpu().numpy()[:, :, :, 0]
    U = repr_np.shape[2]
    orc_sel = np.zeros_like(sel)
    exemptions = 0
    for i, row, pos, L in items:
        e = orc.num_eligible(pos + L - 1, U, w.block, w.n_init, w.window)
        for bi in range(w.batch):
            for h in range(w.n_kv_heads):
                so = orc.score_units(q_cpu[bi, h * G:(h + 1) * G, row:row + L], repr_np[bi, h], e)
                orc_sel[i, bi, h] = orc.topk(so, e, w.top_k)
                exemptions += check_selection(sel[i, bi, h], orc_sel[i, bi, h], so)
    return sel, orc_sel, exemptions


def check_outputs(orc, w, q_cpu, k_cpu, v_cpu, out_gpu, sel_log, points, rope_theta=0.0):
    """points: (index into sel_log, query row, position)."""
    sel = sel_log.cpu().numpy()[:, :, :, 0]
    worst = 0.0
    for i, row, pos in points:
        o_ref, l_ref = orc.attend_all(q_cpu[:, :, row:row + 1], pos, k_cpu, v_cpu, sel[i],
                                      B=w.block, n_init=w.n_init, W=w.window,
                                      rope_theta=rope_theta)
        got = out_gpu[:, :, row:row + 1]
        worst = max(worst, assert_close(got, o_ref, tolerance(q_cpu.dtype, o_ref),
                                        "%s position %d" % (w.name, pos)))
    return worst


def test_fullsize_llama3_32k_encode(orc):
    w, p = run("llama3_8b_32k_encode")
    U = p.U
    check_build(orc, w, p, [(0, 0, 0, 8), (0, 5, U // 2, U // 2 + 8), (0, 7, U - 8, U)])
    q = p.inp["q"].cpu()
    items = [(c, c * w.chunk, c * w.chunk, w.chunk) for c in range(p.n_chunks)]
    check_selections(orc, w, p, q, p.sel_enc, items)
    k, v = p.inp["k"].cpu(), p.inp["v"].cpu()
    pts = [(t // w.chunk, t, t) for t in (0, 5, 127, 128, 4200, 4223, 4224, 4351, 4352, 16383,
                                          16384, 20000, 32767)]
    check_outputs(orc, w, q, k, v, p.out_enc, p.sel_enc, pts)


def test_fullsize_llama3_128k_decode(orc):
    w, p = run("llama3_8b_128k_decode")
    U = p.U
    check_build(orc, w, p, [(0, 0, 0, 8), (3, 7, U - 8, U)])
    qd = p.inp["q_dec"].cpu()
    items = [(s, s, w.n_ctx + s, 1) for s in range(w.decode_steps)]
    check_selections(orc, w, p, qd, p.sel_dec, items)
    k, v = p.inp["k"].cpu(), p.inp["v"].cpu()
    check_outputs(orc, w, qd, k, v, p.out_dec, p.sel_dec,
                  [(s, s, w.n_ctx + s) for s in (0, 1, 128, 255)])


def test_fullsize_llama3_128k_decode_rope(orc):
    """The 128K decode steps with positions inside the working context
    (rope_theta 500,000, Llama-3's base), in the form bench.py --rope-theta
    times (one launch per step): selections re-derived from the oracle's
    scores, sampled outputs against the oracle's re-positioned attention.
    Entries of std 1 instead of 1/sqrt(128): logits of order 10, so that a
    wrong turn moves the softmax weights by far more than the tolerance."""
    theta = 500000.0
    w, p = run("llama3_8b_128k_decode", rope_theta=theta, scale=1.0)
    assert p.fused
    qd = p.inp["q_dec"].cpu()
    items = [(s, s, w.n_ctx + s, 1) for s in range(0, w.decode_steps, 17)]
    check_selections(orc, w, p, qd, p.sel_dec, items)
    k, v = p.inp["k"].cpu(), p.inp["v"].cpu()
    check_outputs(orc, w, qd, k, v, p.out_dec, p.sel_dec,
                  [(s, s, w.n_ctx + s) for s in (0, 1, 128, 255)], rope_theta=theta)


def test_fullsize_llama3_128k_range_build(orc):
    """Streaming unit build at the full size: the last units of the 128K
    context (windows truncated at the end), and the newest units of a
    shorter, ragged context, each written into its rows of a pool."""
    w = synth.WORKLOADS["llama3_8b_128k_decode"]
    p = bench.Pipeline(w)
    U = p.U
    rep = torch.full_like(p.rep_idx, -7)
    repr_ = torch.full_like(p.repr, float("nan"))
    ws = F.workspace(p.cfg, F.INFLLM_CALL_BUILD_RANGE, w.batch, 16)
    F.infllm_build_units_range(p.cfg, p.inp["q"], p.inp["k"], w.n_ctx, U - 16, U, rep, repr_, ws)
    torch.cuda.synchronize()
    check_build(orc, w, p, [(0, 0, U - 8, U), (3, 7, U - 16, U - 8)], rep_idx=rep, repr_=repr_)
    n_mid = 100003
    Um = F.infllm_num_units(p.cfg, n_mid)
    F.infllm_build_units_range(p.cfg, p.inp["q"], p.inp["k"], n_mid, Um - 8, Um, rep, repr_, ws)
    torch.cuda.synchronize()
    check_build(orc, w, p, [(1, 2, Um - 8, Um)], n_ctx=n_mid, rep_idx=rep, repr_=repr_)
    assert torch.isnan(repr_[:, :, :Um - 8]).all() and (rep[:, :, :Um - 8] == -7).all()


def test_fullsize_llama3_1m_decode_recall(orc):
    w, p = run("llama3_8b_1m_decode")
    U = p.U
    planted = p.inp["planted_units"]                        # absolute blocks [b, H_kv, 8]
    j0 = w.n_init // w.block
    pu = int(planted[0, 0, 0]) - j0
    # units across the whole pool (every tenth of the context) as well as a
    # planted unit and the truncated windows at the end
    spread = [(0, 3, f * U // 10, f * U // 10 + 2) for f in (1, 3, 5, 7, 9)]
    spread += [(1, 2, f * U // 10 + 1, f * U // 10 + 3) for f in (0, 2, 4, 6, 8)]
    check_build(orc, w, p, [(0, 0, pu, pu + 2), (1, 6, U - 6, U)] + spread)
    qd = p.inp["q_dec"].cpu()
    items = [(s, s, w.n_ctx + s, 1) for s in range(w.decode_steps)]
    sel, orc_sel, _ = check_selections(orc, w, p, qd, p.sel_dec, items)
    units = (planted - j0).numpy()
    hit_g = np.array([[[np.isin(units[bi, h], sel[s, bi, h]).sum() for h in range(w.n_kv_heads)]
                       for bi in range(w.batch)] for s in range(w.decode_steps)])
    hit_o = np.array([[[np.isin(units[bi, h], orc_sel[s, bi, h]).sum()
                        for h in range(w.n_kv_heads)] for bi in range(w.batch)]
                      for s in range(w.decode_steps)])
    recall_g = hit_g.sum() / (w.decode_steps * units.size)
    recall_o = hit_o.sum() / (w.decode_steps * units.size)
    print("planted-unit recall at 1M: GPU %.4f oracle %.4f" % (recall_g, recall_o))
    assert recall_g == recall_o
    k, v = p.inp["k"].cpu(), p.inp["v"].cpu()
    check_outputs(orc, w, qd, k, v, p.out_dec, p.sel_dec,
                  [(s, s, w.n_ctx + s) for s in (0, 255)])


@pytest.mark.parametrize("name", ["mistral_7b_64k_tokens", "mistral_7b_64k_mean"])
def test_fullsize_mistral_64k(orc, name):
    w, p = run(name)
    U = p.U
    check_build(orc, w, p, [(0, 0, 0, 8), (0, 3, U - 8, U)])
    q, qd = p.inp["q"].cpu(), p.inp["q_dec"].cpu()
    _, _, ex_enc = check_selections(orc, w, p, q, p.sel_enc,
                                    [(c, c * w.chunk, c * w.chunk, w.chunk)
                                     for c in range(p.n_chunks)])
    _, _, ex_dec = check_selections(orc, w, p, qd, p.sel_dec,
                                    [(s, s, w.n_ctx + s, 1) for s in range(w.decode_steps)])
    print("%s: near-tie exemptions %d (encoding) %d (decode)" % (name, ex_enc, ex_dec))
    k, v = p.inp["k"].cpu(), p.inp["v"].cpu()
    check_outputs(orc, w, q, k, v, p.out_enc, p.sel_enc,
                  [(t // w.chunk, t, t) for t in (100, 4300, 40000, 65535)])
    check_outputs(orc, w, qd, k, v, p.out_dec, p.sel_dec,
                  [(s, s, w.n_ctx + s) for s in (0, 200)])


def test_fullsize_llama3_128k_serving_form(orc):
    """The serving form bench.py --stream times, at the 128K decode size:
    ragged lengths, per-sequence positions, units appended as they leave
    each sequence's window.  The appended units against the oracle at the
    context they were built with, the starting pool on samples, and
    sampled decode steps' selections and outputs per sequence."""
    w = synth.WORKLOADS["llama3_8b_128k_decode"]
    p = bench.StreamPipeline(w)
    p.build_all()
    p.step()
    torch.cuda.synchronize()
    G, B = w.group, w.block
    appended = [(s, bi, lo, hi, n) for s, todo in enumerate(p.builds) for bi, lo, hi, n in todo]
    assert len(appended) >= w.batch
    exemptions = 0
    k_cpu = {}
    for s, bi, lo, hi, n in appended[:4] + [(None, 1, p.start[1] - 6, p.start[1], p.lens[1])]:
        h = (bi * 3 + (lo % 5)) % w.n_kv_heads
        k = p.inp["k"][bi, h, :n].cpu()
        qg = p.q_all[bi, h * G:(h + 1) * G, :n].cpu()
        rep_o, repr_o, ks_o = orc.build_tokens(qg, k, n, B, w.n_init, w.window, w.rep_k, lo, hi)
        rep_g = p.layers[0]["rep_idx"][bi, h, lo:hi].cpu().numpy()
        repr_g = p.layers[0]["repr"][bi, h, lo:hi].cpu().numpy()
        for i in range(hi - lo):
            if np.array_equal(rep_g[i], rep_o[i]):
                np.testing.assert_array_equal(repr_g[i], repr_o[i].astype(np.float32))
                continue
            start = (lo + i + w.n_init // B) * B
            by_pos = {start + t: ks_o[i, t] for t in range(B) if np.isfinite(ks_o[i, t])}
            exemptions += check_selection(rep_g[i], rep_o[i], by_pos)
    assert exemptions <= 1
    qd = p.inp["q_dec"].cpu()
    sel = p.sel_dec.cpu().numpy()[:, :, :, 0]
    repr_np = p.layers[0]["repr"].cpu().double().numpy()
    kk, vv = p.inp["k"].cpu(), p.inp["v"].cpu()
    for s in (0, 200, 255):
        for bi in (0, w.batch - 1):
            t = int(p.pos_host[s, bi])
            e = orc.num_eligible(t, p.U, B, w.n_init, w.window)
            for h in (0, w.n_kv_heads - 1):
                so = orc.score_units(qd[bi, h * G:(h + 1) * G, s:s + 1], repr_np[bi, h], e)
                check_selection(sel[s, bi, h], orc.topk(so, e, w.top_k), so)
            o_ref, _ = orc.attend_all(qd[bi:bi + 1, :, s:s + 1], t, kk[bi:bi + 1], vv[bi:bi + 1],
                                      sel[s, bi:bi + 1], B=B, n_init=w.n_init, W=w.window)
            assert_close(p.out_dec[bi:bi + 1, :, s:s + 1], o_ref,
                         tolerance(torch.bfloat16, o_ref), "serving step %d sequence %d" % (s, bi))
