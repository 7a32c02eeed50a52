"""Helpers for the GPU parity tests: run each C-ABI stage through the ctypes
binding and compare with the oracle under the stated rules.

Selection rule (near ties): the GPU and oracle selections must have the same
size and may differ only in units (or keys) whose oracle score lies within
1e-5 relative of the oracle's k-th kept score -- the k/k+1 near-tie
exemption, generalised to multi-way ties.  Downstream stages are compared on
the GPU's own upstream output, so one tie cannot cascade.

Tolerances: fp32 workloads 1e-4 absolute; bf16 workloads 2e-2 absolute, and
additionally 8e-3 of the largest reference magnitude (the output is rounded
to bf16, 2^-9 relative, and bf16 MFMA products round P and the inputs'
products exactly, so errors stay far below that).
"""
from __future__ import annotations

import numpy as np
import torch

from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth

NEAR_TIE_REL = 1e-5


def cfg_of(w: synth.Workload, **over) -> F.infllm_config:
    kw = dict(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
              block=w.block, n_init=w.n_init, window=w.window, rep_k=w.rep_k, top_k=w.top_k,
              rep_mode=F.INFLLM_REP_MEAN if w.rep_mode == "mean" else F.INFLLM_REP_TOKENS,
              dtype=F.INFLLM_F32 if w.dtype == "f32" else F.INFLLM_BF16)
    kw.update(over)
    return F.make_config(**kw)


def tolerance(dtype: torch.dtype, ref: np.ndarray) -> float:
    if dtype == torch.float32:
        return 1e-4
    return min(2e-2, 8e-3 * float(np.abs(ref).max()) + 1e-6)


# ------------------------------------------------------------------ GPU stages
def gpu_build(cfg, q, k, n_ctx):
    b = k.shape[0]
    U = F.infllm_num_units(cfg, n_ctx)
    repr_ = torch.empty((b, cfg.n_kv_heads, U, cfg.head_dim), dtype=torch.float32, device=k.device)
    rep_idx = None
    if cfg.rep_mode == F.INFLLM_REP_TOKENS:
        rep_idx = torch.empty((b, cfg.n_kv_heads, U, cfg.rep_k), dtype=torch.int32, device=k.device)
    ws = F.workspace(cfg, F.INFLLM_CALL_BUILD, b, n_ctx, device=k.device)
    F.infllm_build_units(cfg, q, k, n_ctx, rep_idx, repr_, ws)
    return rep_idx, repr_


def gpu_score(cfg, q, q_off, q_pos, L, n_chunks, repr_):
    b = q.shape[0]
    scores = torch.empty((b, cfg.n_kv_heads, n_chunks, repr_.shape[2]), dtype=torch.float32,
                         device=q.device)
    ws = F.workspace(cfg, F.INFLLM_CALL_SCORE, b, 0, L, n_chunks, device=q.device)
    F.infllm_score_units(cfg, q, q_off, q_pos, L, n_chunks, repr_, scores, ws)
    return scores


def gpu_topk(cfg, scores):
    b, _, nc, _ = scores.shape
    sel = torch.empty((b, cfg.n_kv_heads, nc, cfg.top_k), dtype=torch.int32, device=scores.device)
    F.infllm_topk_units(cfg, scores, sel)
    return sel


def gpu_attend(cfg, q, q_off, q_pos, L, n_chunks, k, v, sel, with_lse=True):
    b = q.shape[0]
    n = L * n_chunks
    out = torch.empty((b, cfg.n_q_heads, n, cfg.head_dim), dtype=q.dtype, device=q.device)
    lse = torch.empty((b, cfg.n_q_heads, n), dtype=torch.float32, device=q.device) if with_lse \
        else None
    ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, L, n_chunks, device=q.device)
    F.infllm_attend(cfg, q, q_off, q_pos, L, n_chunks, k, v, sel, out, lse, 0, ws)
    return out, lse


# ------------------------------------------------------------------ comparisons
def check_selection(gpu_sel, orc_sel, orc_scores, rel=NEAR_TIE_REL) -> bool:
    """gpu_sel / orc_sel: 1-D index lists with -1 pads; orc_scores indexed by
    the same ids.  Returns True if a near-tie exemption was needed."""
    g = set(int(x) for x in np.asarray(gpu_sel) if x >= 0)
    o = set(int(x) for x in np.asarray(orc_sel) if x >= 0)
    assert len(g) == len(o), (sorted(g), sorted(o))
    assert sorted(np.asarray(gpu_sel)[:len(g)].tolist()) == np.asarray(gpu_sel)[:len(g)].tolist()
    assert all(x == -1 for x in np.asarray(gpu_sel)[len(g):])
    if g == o:
        return False
    tau = min(float(orc_scores[u]) for u in o)
    for u in g ^ o:
        assert abs(float(orc_scores[u]) - tau) <= rel * abs(tau), (u, orc_scores[u], tau)
    return True


def check_rep_idx(gpu_rep, orc_rep, orc_key_scores, B, n_init):
    """Per unit: rep_idx sets equal up to near ties of the oracle key scores.
    Returns the (b, h, u) triples where an exemption was used."""
    ex = []
    gb, ob = np.asarray(gpu_rep), np.asarray(orc_rep)
    for idx in np.ndindex(ob.shape[:-1]):
        go, oo = gb[idx], ob[idx]
        if np.array_equal(go, oo):
            continue
        ks = orc_key_scores[idx]
        block_start = (idx[-1] + n_init // B) * B
        by_pos = {block_start + s: ks[s] for s in range(B) if np.isfinite(ks[s])}
        if check_selection(go, oo, by_pos):
            ex.append(idx)
    return ex


def assert_close(gpu, ref, tol, what):
    g = gpu.float().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    err = np.abs(g.astype(np.float64) - ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, "%s: max abs error %.3e > %.3e" % (what, worst, tol)
    return worst
