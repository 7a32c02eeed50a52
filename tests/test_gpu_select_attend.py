"""infllm_select_attend (one decode step in one launch where the shapes
allow): scores and selections bit-identical to infllm_select_units, outputs
against the oracle on the GPU's selection and close to infllm_attend on it
(the attention is split over workgroups differently, so only fp32 rounding
may differ), repeated calls on one workspace, positions per sequence
(including ones that do not fit the KV buffer), and the shapes that take the
separate calls."""
import numpy as np
import pytest
import torch

from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth
from gpu_helpers import assert_close, cfg_of, check_selection, gpu_build, tolerance

pytestmark = pytest.mark.gpu


def separate(cfg, q, q_off, q_pos, n_pos, repr_, k, v, pos=None):
    """The reference: infllm_select_units, then infllm_attend(_varlen)."""
    b, U = q.shape[0], repr_.shape[2]
    scores = torch.empty((b, cfg.n_kv_heads, n_pos, U), dtype=torch.float32, device="cuda")
    sel = torch.empty((b, cfg.n_kv_heads, n_pos, cfg.top_k), dtype=torch.int32, device="cuda")
    F.infllm_select_units(cfg, q, q_off, q_pos, 1, n_pos, repr_, scores, sel, pos=pos,
                          ws=F.workspace(cfg, F.INFLLM_CALL_SELECT, b, 0, 1, n_pos))
    out = torch.empty((b, cfg.n_q_heads, n_pos, cfg.head_dim), dtype=q.dtype, device="cuda")
    lse = torch.empty((b, cfg.n_q_heads, n_pos), dtype=torch.float32, device="cuda")
    aws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, 1, n_pos)
    if pos is None:
        F.infllm_attend(cfg, q, q_off, q_pos, 1, n_pos, k, v, sel, out, lse, 0, aws)
    else:
        F.infllm_attend_varlen(cfg, q, q_off, pos, 1, n_pos, k, v, sel, out, lse, 0, aws)
    return scores, sel, out, lse


def fused(cfg, q, q_off, q_pos, n_pos, repr_, k, v, ws, pos=None):
    b, U = q.shape[0], repr_.shape[2]
    scores = torch.full((b, cfg.n_kv_heads, n_pos, U), 7.0, dtype=torch.float32, device="cuda")
    sel = torch.full((b, cfg.n_kv_heads, n_pos, cfg.top_k), -5, dtype=torch.int32, device="cuda")
    out = torch.zeros((b, cfg.n_q_heads, n_pos, cfg.head_dim), dtype=q.dtype, device="cuda")
    lse = torch.zeros((b, cfg.n_q_heads, n_pos), dtype=torch.float32, device="cuda")
    F.infllm_select_attend(cfg, q, q_off, q_pos, n_pos, repr_, k, v, scores, sel, out, lse,
                           pos=pos, ws=ws)
    return scores, sel, out, lse


def compare(orc, cfg, got, ref, q_c, q_off, t_list, k_c, v_c, bad=(), rope_theta=0.0):
    """got (fused) against ref (separate calls) and the oracle; t_list[b] is
    the position of query row q_off of sequence b; q_c, k_c, v_c: the inputs
    on the host."""
    s, sel, out, lse = got
    rs, rsel, rout, rlse = ref
    torch.cuda.synchronize()
    assert torch.equal(sel, rsel)
    good = [b for b in range(len(t_list)) if b not in bad]
    for b in good:
        assert torch.equal(s[b], rs[b])
    for b in bad:
        assert torch.isnan(out[b].float()).all() and torch.isnan(lse[b]).all()
    sg, selg = s.cpu().double().numpy(), sel.cpu().numpy()
    n_pos = sel.shape[2]
    for b in good:
        for idx in np.ndindex(cfg.n_kv_heads, n_pos):
            row = sg[(b,) + idx]
            e = int(np.isfinite(row).sum())
            assert e == orc.num_eligible(t_list[b] + idx[1], row.size, cfg.block, cfg.n_init,
                                         cfg.window)
            assert selg[(b,) + idx].tolist() == orc.topk(row, e, cfg.top_k).tolist()
        for c in range(n_pos):
            o_ref, l_ref = orc.attend_all(q_c[b:b + 1, :, q_off + c:q_off + c + 1],
                                          t_list[b] + c, k_c[b:b + 1], v_c[b:b + 1],
                                          selg[b:b + 1, :, c], B=cfg.block, n_init=cfg.n_init,
                                          W=cfg.window, rope_theta=rope_theta)
            tol = tolerance(out.dtype, o_ref)
            assert_close(out[b:b + 1, :, c:c + 1], o_ref, tol, "seq %d pos %d" % (b, c))
            assert_close(lse[b:b + 1, :, c:c + 1], l_ref, 1e-3, "lse seq %d pos %d" % (b, c))
            assert_close(out[b:b + 1, :, c:c + 1], rout[b:b + 1, :, c:c + 1].float().cpu().numpy(),
                         tol, "vs separate calls, seq %d pos %d" % (b, c))
            assert_close(lse[b:b + 1, :, c:c + 1], rlse[b:b + 1, :, c:c + 1].cpu().numpy(), 1e-4,
                         "lse vs separate calls, seq %d pos %d" % (b, c))


def test_decode_steps_one_workspace(orc):
    """Consecutive decode steps on built units, all on one workspace."""
    w = synth.WORKLOADS["llama3_8b_128k_decode"].replace(n_ctx=6144, batch=2, n_q_heads=8,
                                                         n_kv_heads=2, decode_steps=5, top_k=8,
                                                         window=1024)
    cfg = cfg_of(w)
    inp = synth.make_inputs(w)
    dev = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    _, repr_g = gpu_build(cfg, dev["q"], dev["k"], w.n_ctx)
    U = repr_g.shape[2]
    ws = F.workspace(cfg, F.INFLLM_CALL_SELECT_ATTEND, w.batch, U, 1, 1)
    for s in range(w.decode_steps):
        t = w.n_ctx + s
        got = fused(cfg, dev["q_dec"], s, t, 1, repr_g, dev["k"], dev["v"], ws)
        ref = separate(cfg, dev["q_dec"], s, t, 1, repr_g, dev["k"], dev["v"])
        compare(orc, cfg, got, ref, inp["q_dec"], s, [t] * w.batch, inp["k"], inp["v"])
        # the oracle's own scores pick the same units (up to near ties)
        sg = got[1].cpu().numpy()
        e = orc.num_eligible(t, U, w.block, w.n_init, w.window)
        G = w.group
        rn = repr_g.cpu().double().numpy()
        for bi in range(w.batch):
            for h in range(w.n_kv_heads):
                so = orc.score_units(inp["q_dec"][bi, h * G:(h + 1) * G, s:s + 1], rn[bi, h], e)
                check_selection(sg[bi, h, 0], orc.topk(so, e, w.top_k), so)


ANY_PLAN = "any"   # a plan whose shape the test does not fix


# (Hq, Hkv, d, U, k_m, n_pos, W, n_init, varlen, dtype, plan): plan is the
# one-launch shape infllm_step_plan must report, (workgroups per row,
# scoring workgroups, units each), or None for the two separate calls
SHAPES = [
    (8, 2, 128, 47, 8, 1, 1024, 128, False, "bf16", (63, 1, 64)),      # one scorer per row
    (4, 4, 128, 300, 16, 2, 512, 128, False, "bf16", (15, 5, 64)),     # G = 1, two positions
    (8, 4, 64, 200, 6, 3, 384, 100, False, "bf16", (9, 4, 64)),       # G = 2, d = 64, sinks not B-aligned
    (16, 2, 128, 100, 4, 1, 512, 128, True, "bf16", (63, 2, 64)),      # G = 8, a position per sequence
    (8, 2, 128, 1024, 32, 1, 1024, 128, False, "bf16", (63, 16, 64)),  # 512 candidates per row
    (8, 1, 128, 2048, 32, 1, 512, 128, False, "bf16", (64, 32, 64)),   # 32 scorers
    (8, 2, 128, 1500, 32, 8, 512, 128, False, "bf16", (15, 12, 128)),  # 128 units per scorer
    (8, 2, 128, 1500, 32, 16, 512, 128, False, "bf16", (11, 8, 192)),  # 192 units per scorer
    (4, 2, 128, 4000, 32, 1, 512, 128, False, "bf16", None),  # more scores than one search: two calls
    (4, 2, 128, 300, 8, 16, 512, 128, False, "bf16", (3, 2, 192)),     # few workgroups per row
    (4, 2, 128, 30, 40, 1, 512, 128, False, "bf16", (63, 1, 64)),      # k_m > units
    (4, 2, 128, 600, 256, 1, 512, 128, False, "bf16", (63, 10, 64)),   # the largest k_m
    (8, 2, 128, 64, 2, 1, 4096, 128, False, "bf16", (63, 1, 64)),      # nearly all keys local
    (32, 8, 128, 300, 8, 32, 512, 128, False, "bf16", (3, 2, 256)),    # 2,048 workgroups: more than fit at once
    (4, 2, 128, 4095, 256, 1, 512, 128, False, "bf16", None),          # 4,096 candidates: separate calls
    (2, 1, 64, 40, 4, 1, 512, 64, False, "f32", None),                 # fp32: separate calls
]


@pytest.mark.parametrize("Hq,Hkv,d,U,k_m,n_pos,W,n_init,varlen,dt,plan", SHAPES)
def test_select_attend_shapes(orc, Hq, Hkv, d, U, k_m, n_pos, W, n_init, varlen, dt, plan):
    run_shape(orc, Hq, Hkv, d, U, k_m, n_pos, W, n_init, varlen, dt, plan)


def run_shape(orc, Hq, Hkv, d, U, k_m, n_pos, W, n_init, varlen, dt, plan, cut=False,
              rope_theta=0.0):
    """Random unit representations and K/V; the last position sees every unit
    eligible, a second sequence (varlen) sits mid-context.  Two calls in a
    row on one workspace, bit for bit equal; no wait hits its bound.  cut:
    the plan must have every slice publish fewer candidates than units.
    rope_theta > 0: positions inside the working context, q and k of std 1
    (logits of order 10, so that a wrong turn shows)."""
    b, B = 2, 128
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B, n_init=n_init,
                        window=W, rep_k=4, top_k=k_m,
                        dtype=F.INFLLM_BF16 if dt == "bf16" else F.INFLLM_F32,
                        rope_theta=rope_theta)
    got_plan = F.infllm_step_plan(cfg, b, U, n_pos)
    if plan is None:
        assert got_plan["fused"] == 0
    elif plan is not ANY_PLAN:
        assert (got_plan["n_splits"], got_plan["s_score"], got_plan["units_per"]) == plan
    if cut:
        assert got_plan["fused"] == 1 and got_plan["cand"] < got_plan["units_per"], got_plan
    gen = torch.Generator().manual_seed(U * 31 + k_m + n_pos)
    n_units_ctx = U + n_init // B                       # blocks before the window
    t0 = n_units_ctx * B + W + 17                       # every unit eligible
    cap = t0 + n_pos + 5
    scale = 1.0 if rope_theta > 0 else d ** -0.5
    q = (torch.randn((b, Hq, n_pos + 2, d), generator=gen) * scale).to(dtype)
    k = (torch.randn((b, Hkv, cap, d), generator=gen) * scale).to(dtype)
    v = (torch.randn((b, Hkv, cap, d), generator=gen) * scale).to(dtype)
    repr_ = torch.randn((b, Hkv, U, d), generator=gen)
    qg, kg, vg, rg = q.cuda(), k.cuda(), v.cuda(), repr_.cuda()
    t_list = [t0, t0]
    pos = None
    if varlen:
        t_list = [t0, B * (U // 2) + W + n_init]
        pos = torch.tensor(t_list, dtype=torch.int64).cuda()
    ws = F.workspace(cfg, F.INFLLM_CALL_SELECT_ATTEND, b, U, 1, n_pos)
    ref = separate(cfg, qg, 2, t0, n_pos, rg, kg, vg, pos=pos)
    first = None
    for _ in range(2):
        got = fused(cfg, qg, 2, t0, n_pos, rg, kg, vg, ws, pos=pos)
        compare(orc, cfg, got, ref, q, 2, t_list, k, v, rope_theta=rope_theta)
        if first is None:
            first = got
        else:   # the same bits on the second call (fixed merge order)
            assert all(torch.equal(x, y) for x, y in zip(first, got))
    assert F.infllm_workspace_status(ws) == 0
    return ws


# positions inside the working context (rope_theta > 0): one launch with at
# most two workgroups per CU for up to 4 query heads per KV head at head_dim
# 128, the two calls otherwise
ROPE_SHAPES = [
    (4, 4, 128, 300, 16, 2, 512, 128, False, "bf16", (15, 5, 64)),    # G = 1, two positions
    (8, 4, 128, 200, 6, 3, 384, 100, True, "bf16", (9, 4, 64)),       # G = 2, sinks not B-aligned
    (8, 2, 128, 1500, 32, 8, 512, 128, False, "bf16", (15, 12, 128)), # G = 4, eight positions
    (8, 2, 128, 600, 256, 1, 512, 128, True, "bf16", (63, 10, 64)),   # the largest k_m
    (16, 2, 128, 100, 4, 1, 512, 128, True, "bf16", None),            # G = 8: the two calls
    (8, 4, 64, 200, 6, 1, 384, 100, False, "bf16", None),             # d = 64: the two calls
]


@pytest.mark.parametrize("Hq,Hkv,d,U,k_m,n_pos,W,n_init,varlen,dt,plan", ROPE_SHAPES)
def test_select_attend_rope_shapes(orc, Hq, Hkv, d, U, k_m, n_pos, W, n_init, varlen, dt, plan):
    run_shape(orc, Hq, Hkv, d, U, k_m, n_pos, W, n_init, varlen, dt, plan, rope_theta=500000.0)


# one launch for rows with more scores than one search takes (as at the
# 1M-token context): each slice publishes only its best k_m.  The library
# takes this form only with the split count set by hand, read once per
# process, so it runs in a child process.
CUT_SHAPES = [
    (4, 2, 128, 4000, 32, 1, 512, 128, False, "bf16"),    # best 32 of 128 per slice
    (8, 1, 128, 8191, 32, 1, 512, 128, True, "bf16"),     # 8,191 units: best 32 of 256 per slice
]


def test_select_attend_candidate_cut():
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys\n"
            "sys.path[:0] = [%r, %r]\n"
            "from oracle import oracle as orc\n"
            "import test_gpu_select_attend as t\n"
            "for sh in t.CUT_SHAPES:\n"
            "    print('shape', sh, flush=True)\n"
            "    t.run_shape(orc, *sh, plan=t.ANY_PLAN, cut=True)\n"
            "print('ok', flush=True)\n") % (here, os.path.dirname(here))
    env = dict(os.environ, INFLLM_STEP_SPLITS="48")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


# The attention workgroups' bounded spin for the selector set to zero: every
# one that finds its row's selection unpublished selects the row itself
# (the path that keeps the step independent of the selector being
# dispatched); the selector may then arrive last and clear the row.  Read
# once per process, so it runs in a child process.
SELF_SELECT_SHAPES = [
    (8, 2, 128, 1024, 32, 1, 1024, 128, False, "bf16"),   # 16 scorers, 512 candidates
    (16, 2, 128, 100, 4, 1, 512, 128, True, "bf16"),      # G = 8, a position per sequence
    (4, 2, 128, 600, 256, 1, 512, 128, False, "bf16"),    # the largest k_m
    (32, 8, 128, 300, 8, 32, 512, 128, False, "bf16"),    # 2,048 workgroups
    (8, 4, 64, 200, 6, 3, 384, 100, False, "bf16"),       # d = 64, sinks not B-aligned
]


def test_select_attend_self_selection():
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys\n"
            "sys.path[:0] = [%r, %r]\n"
            "from oracle import oracle as orc\n"
            "import test_gpu_select_attend as t\n"
            "for sh in t.SELF_SELECT_SHAPES:\n"
            "    print('shape', sh, flush=True)\n"
            "    ws = t.run_shape(orc, *sh, plan=t.ANY_PLAN)\n"
            "    print('self-selected rows', int(ws[4:8].view(t.torch.int32)[0]), flush=True)\n"
            "print('ok', flush=True)\n") % (here, os.path.dirname(here))
    env = dict(os.environ, INFLLM_STEP_PRESPIN="0")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
    # the path ran: some rows were selected by attention workgroups
    n_self = [int(x.split()[-1]) for x in r.stdout.splitlines() if x.startswith("self-selected")]
    assert len(n_self) == len(SELF_SELECT_SHAPES) and sum(n_self) > 0, r.stdout


def test_select_attend_bad_positions(orc):
    """A position per sequence where two do not fit the KV buffer: NaN rows
    there, the others as the separate calls; then valid positions again on
    the same workspace."""
    Hq, Hkv, d, U, k_m, W, n_init, B, b = 8, 2, 128, 120, 8, 512, 128, 128, 4
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B, n_init=n_init,
                        window=W, rep_k=4, top_k=k_m)
    gen = torch.Generator().manual_seed(5)
    cap = (U + 1) * B + W + 20
    q = (torch.randn((b, Hq, 1, d), generator=gen) * 0.09).to(torch.bfloat16)
    k = (torch.randn((b, Hkv, cap, d), generator=gen) * 0.09).to(torch.bfloat16)
    v = (torch.randn((b, Hkv, cap, d), generator=gen) * 0.09).to(torch.bfloat16)
    rg = torch.randn((b, Hkv, U, d), generator=gen).cuda()
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    ws = F.workspace(cfg, F.INFLLM_CALL_SELECT_ATTEND, b, U, 1, 1)
    for t_list, bad in (([cap - 1, -1, cap, 3000], {1, 2}), ([cap - 1, 9000, 700, 3000], set())):
        pos = torch.tensor(t_list, dtype=torch.int64).cuda()
        got = fused(cfg, qg, 0, 0, 1, rg, kg, vg, ws, pos=pos)
        ref = separate(cfg, qg, 0, 0, 1, rg, kg, vg, pos=pos)
        compare(orc, cfg, got, ref, q, 0, t_list, k, v, bad=bad)
