"""GPU parity of the serving form (bench.StreamPipeline): ragged sequence
lengths, a device position per sequence, units added to every layer's pool
as they leave each sequence's window.  Against the oracle: every unit of
the final pools, built from the queries up to the position where it joined
(or from the whole starting context), and sampled decode steps' selections
and attention outputs, per sequence at its own position."""
import numpy as np
import pytest
import torch

import bench
from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth
from gpu_helpers import assert_close, check_selection, tolerance

pytestmark = pytest.mark.gpu


def test_stream_pipeline(orc):
    w = synth.WORKLOADS["llama3_8b_128k_decode"].replace(n_ctx=6144, batch=3, n_q_heads=8,
                                                         n_kv_heads=2, decode_steps=300,
                                                         top_k=8, window=1024)
    p = bench.StreamPipeline(w, layers=2)
    p.build_all()
    p.step()
    torch.cuda.synchronize()
    assert p.n_builds >= 6 and len(set(p.lens)) == w.batch
    B, G = w.block, w.group
    # when each unit joined: (n_ctx it was built with) per sequence
    built_at = []
    for bi in range(w.batch):
        m = {u: p.lens[bi] for u in range(p.start[bi])}
        for todo in p.builds:
            for b2, lo, hi, n in todo:
                if b2 == bi:
                    m.update({u: n for u in range(lo, hi)})
        built_at.append(m)
    qa = p.q_all.cpu()
    exemptions = 0
    for li, ly in enumerate(p.layers):
        k_cpu = ly["k"].cpu()
        rep = ly["rep_idx"].cpu().numpy()
        rr = ly["repr"].cpu().numpy()
        for bi in range(w.batch):
            by_n = {}
            for u, n in built_at[bi].items():
                by_n.setdefault(n, []).append(u)
            for n, units in by_n.items():
                lo, hi = min(units), max(units) + 1
                assert hi - lo == len(units)
                for h in range(w.n_kv_heads):
                    rep_o, repr_o, ks_o = orc.build_tokens(qa[bi, h * G:(h + 1) * G, :n],
                                                           k_cpu[bi, h, :n], n, B, w.n_init,
                                                           w.window, w.rep_k, lo, hi)
                    for i in range(hi - lo):
                        g = rep[bi, h, lo + i]
                        if np.array_equal(g, rep_o[i]):
                            np.testing.assert_array_equal(rr[bi, h, lo + i],
                                                          repr_o[i].astype(np.float32))
                            continue
                        start = (lo + i + w.n_init // B) * B
                        by_pos = {start + s: ks_o[i, s] for s in range(B)
                                  if np.isfinite(ks_o[i, s])}
                        exemptions += check_selection(g, rep_o[i], by_pos)
            # rows never built stay as allocated
            last = max(built_at[bi]) + 1
            assert (rep[bi, :, last:] == -1).all()
    assert exemptions <= 2
    # sampled steps: selection from the oracle's fp64 scores on the GPU's
    # pool (near-tie rule) and attention outputs, per sequence
    qd = p.inp["q_dec"].cpu()
    sel = p.sel_dec.cpu().numpy()[:, :, :, 0]
    k0, v0 = p.layers[0]["k"].cpu(), p.layers[0]["v"].cpu()
    k1, v1 = p.layers[1]["k"].cpu(), p.layers[1]["v"].cpu()
    for s in (0, 1, 150, 299):
        li = s % len(p.layers)
        repr_np = p.layers[li]["repr"].cpu().double().numpy()
        kk, vv = (k0, v0) if li == 0 else (k1, v1)
        for bi in range(w.batch):
            t = int(p.pos_host[s, bi])
            e = orc.num_eligible(t, p.U, B, w.n_init, w.window)
            for h in range(w.n_kv_heads):
                so = orc.score_units(qd[bi, h * G:(h + 1) * G, s:s + 1], repr_np[bi, h], e)
                check_selection(sel[s, bi, h], orc.topk(so, e, w.top_k), so)
            o_ref, _ = orc.attend_all(qd[bi:bi + 1, :, s:s + 1], t, kk[bi:bi + 1], vv[bi:bi + 1],
                                      sel[s, bi:bi + 1], B=B, n_init=w.n_init, W=w.window)
            assert_close(p.out_dec[bi:bi + 1, :, s:s + 1], o_ref, tolerance(torch.bfloat16, o_ref),
                         "stream step %d sequence %d" % (s, bi))
