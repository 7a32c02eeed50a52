"""GPU parity of the attention with rotary positions inside the working
context (rope_theta > 0) against the oracle's re-positioning (InfLLM Guide,
"Operational Checklist", RoPE item).  Covered: the MFMA chunk path (G = 4
and 8, sinks not a multiple of B), the vector path (fp32, d = 64, decode
rows), queries before n_init, unit keys past the chunk's first local place,
empty slots and repeated ids, a position near 300K (angle reduction), the
per-sequence-position form and the decode step.  Random q and k stand for
vectors turned at their absolute positions: the re-positioning is linear, so
any vectors check it."""
import numpy as np
import pytest
import torch

from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth
from gpu_helpers import assert_close, cfg_of, gpu_attend, tolerance

pytestmark = pytest.mark.gpu

LL = synth.WORKLOADS["llama3_8b_32k_encode"]
# q, k, v entries of std 1 (scale 1): logits of order 1, so that a wrong
# turn moves the softmax weights by far more than the tolerance (at the
# Llama-shaped 1/sqrt(d) the weights are nearly uniform whatever the turn)
CASES = {
    # MFMA path, G=4: window a multiple of B
    "bf16_g4": (LL.replace(n_ctx=2304, n_q_heads=8, n_kv_heads=2, window=384, top_k=5,
                           chunk=128, scale=1.0), 10000.0),
    # MFMA path, G=8, sinks 100 (unit 0 starts past them), window not a multiple of B
    "bf16_g8_ragged": (LL.replace(n_ctx=2200, n_q_heads=8, n_kv_heads=1, window=300, n_init=100,
                                  top_k=6, chunk=96, scale=1.0), 500000.0),
    # vector path, fp32, G=1, d=64
    "f32_g1": (synth.WORKLOADS["tiny_f32"].replace(n_ctx=1536), 10000.0),
    # vector path, bf16, G=2, d=64
    "bf16_g2_d64": (LL.replace(n_ctx=1800, n_q_heads=4, n_kv_heads=2, head_dim=64, window=256,
                               top_k=3, chunk=64, scale=1.0), 10000.0),
}


@pytest.fixture(scope="module")
def data():
    cache = {}

    def get(name):
        if name not in cache:
            w, theta = CASES[name]
            inp = synth.make_inputs(w)
            dev = {k: v.cuda() for k, v in inp.items() if k in ("q", "k", "v")}
            cache[name] = (w, theta, inp, dev)
        return cache[name]
    return get


def selections(orc, w, t0s, L, seed):
    """sel [b, H_kv, len(t0s), k_m]: per chunk, distinct eligible units in
    random slots with empty slots between, the newest eligible unit always in
    (its keys reach the chunk's first local place) and the first id repeated
    in the last slot when there is room."""
    g = np.random.default_rng(seed)
    U = orc.num_units(w.n_ctx, w.block, w.n_init)
    k_m = w.top_k
    sel = np.full((w.batch, w.n_kv_heads, len(t0s), k_m), -1, np.int32)
    for c, t0 in enumerate(t0s):
        e = orc.num_eligible(t0 + L - 1, U, w.block, w.n_init, w.window)
        for bi in range(w.batch):
            for h in range(w.n_kv_heads):
                n = min(e, k_m - 2) if k_m > 2 else min(e, k_m)
                if n <= 0:
                    continue
                ids = [e - 1] + [int(x) for x in g.choice(e - 1, size=n - 1, replace=False)] \
                    if e > 1 else [0]
                slots = np.sort(g.choice(k_m - 1 if k_m > 1 else 1, size=len(ids),
                                         replace=False))
                for s, u in zip(slots, ids):
                    sel[bi, h, c, s] = u
                if k_m > 1 and sel[bi, h, c, -1] < 0:
                    sel[bi, h, c, -1] = ids[0]
    return sel


def mfma_rounding_bound(w, q_chunk, k, t0, L):
    """[b, H_q, L] bound on the logit error that rounding turned vectors to
    bf16 adds on the MFMA chunk path: each turned key element is off by at
    most 2^-9 of itself, so q.k' moves by at most 2^-9 sum_c |q_c k'_c| <=
    2^-9 sum_pairs |q_pair| |k_pair| (Cauchy-Schwarz per rotary pair; a
    turn keeps pair lengths), over sqrt(d); queries before n_init are turned
    and rounded too (twice the bound).  Taken over every key of the context,
    a superset of the attended ones."""
    d = w.head_dim
    h = d // 2
    G = w.n_q_heads // w.n_kv_heads
    qf = q_chunk.double().numpy()          # [b, H_q, L, d], positions t0 ..
    kf = k[:, :, :t0 + L].double().numpy()
    qn = np.hypot(qf[..., :h], qf[..., h:])
    kn = np.hypot(kf[..., :h], kf[..., h:])
    bound = np.zeros(qf.shape[:3])
    for bi in range(qf.shape[0]):
        for hq in range(qf.shape[1]):
            bound[bi, hq] = (qn[bi, hq] @ kn[bi, hq // G].T).max(axis=1)
    early = (t0 + np.arange(L)) < w.n_init
    return 2.0 ** -9 * bound / np.sqrt(d) * np.where(early, 2.0, 1.0) * (1 + 2.0 ** -7)


def check_chunks(orc, w, theta, inp, out, lse, sel, t0s, L, what, only=None):
    """Chunk c of out / lse against the oracle, for c in `only` (all by
    default).  LSE: 1e-3 (bf16) / 1e-4 (fp32), plus on the MFMA chunk path
    (bf16, d = 128, chunks of >= 16) the bound of mfma_rounding_bound."""
    mfma = inp["q"].dtype == torch.bfloat16 and w.head_dim == 128 and L >= 16
    for c, t0 in enumerate(t0s):
        if only is not None and c not in only:
            continue
        o_ref, l_ref = orc.attend_all(inp["q"][:, :, t0:t0 + L], t0, inp["k"], inp["v"],
                                      sel[:, :, c], B=w.block, n_init=w.n_init, W=w.window,
                                      rope_theta=theta)
        tol = tolerance(inp["q"].dtype, o_ref)
        assert_close(out[:, :, c * L:(c + 1) * L], o_ref, tol, "%s chunk %d out" % (what, c))
        l_tol = 1e-4 if inp["q"].dtype == torch.float32 else 1e-3
        l_gpu = lse[:, :, c * L:(c + 1) * L].cpu().numpy().astype(np.float64)
        err = np.abs(l_gpu - l_ref)
        if mfma:
            bound = l_tol + mfma_rounding_bound(w, inp["q"][:, :, t0:t0 + L], inp["k"], t0, L)
            assert (err <= bound).all(), "%s chunk %d lse: worst excess %.3e" % (
                what, c, float((err - bound).max()))
        else:
            assert err.max() <= l_tol, "%s chunk %d lse: %.3e" % (what, c, float(err.max()))


@pytest.mark.parametrize("name", list(CASES))
def test_rope_chunks(orc, data, name):
    """Every chunk of the context from position 0 (the first holds queries
    before n_init) in one call; the first two, a middle one and the last two
    checked (the oracle turns every key per query)."""
    w, theta, inp, dev = data(name)
    L = w.chunk
    n_chunks = w.n_ctx // L
    t0s = [c * L for c in range(n_chunks)]
    sel = selections(orc, w, t0s, L, 1)
    cfg = cfg_of(w, rope_theta=theta)
    out, lse = gpu_attend(cfg, dev["q"], 0, 0, L, n_chunks, dev["k"], dev["v"],
                          torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    check_chunks(orc, w, theta, inp, out, lse, sel, t0s, L, name,
                 only={0, 1, n_chunks // 2, n_chunks - 2, n_chunks - 1})
    # not vacuous: the last chunk without re-positioning is far off
    c, t0 = n_chunks - 1, t0s[-1]
    o_plain, _ = orc.attend_all(inp["q"][:, :, t0:t0 + L], t0, inp["k"], inp["v"], sel[:, :, c],
                                B=w.block, n_init=w.n_init, W=w.window)
    gap = float(np.abs(out[:, :, c * L:].float().cpu().numpy() - o_plain).max())
    assert gap > 10 * tolerance(inp["q"].dtype, o_plain), gap


@pytest.mark.parametrize("name", list(CASES))
def test_rope_decode_rows(orc, data, name):
    """Single positions (the decode form, vector path): early ones before
    n_init and late ones with units."""
    w, theta, inp, dev = data(name)
    cfg = cfg_of(w, rope_theta=theta)
    for t_first, n in ((0, 3), (w.n_init - 1, 2), (w.n_ctx - 6, 6)):
        t0s = [t_first + i for i in range(n)]
        sel = selections(orc, w, t0s, 1, 2 + t_first)
        out, lse = gpu_attend(cfg, dev["q"], t_first, t_first, 1, n, dev["k"], dev["v"],
                              torch.from_numpy(sel).cuda())
        torch.cuda.synchronize()
        check_chunks(orc, w, theta, inp, out, lse, sel, t0s, 1, "%s t=%d" % (name, t_first))


def test_rope_off_matches_plain(orc, data):
    """rope_theta 0 is the plain attention, bit for bit."""
    w, _, inp, dev = data("bf16_g4")
    L = w.chunk
    t0 = w.n_ctx - L
    sel = torch.from_numpy(selections(orc, w, [t0], L, 3)).cuda()
    a, la = gpu_attend(cfg_of(w), dev["q"], t0, t0, L, 1, dev["k"], dev["v"], sel)
    b, lb = gpu_attend(cfg_of(w, rope_theta=0.0), dev["q"], t0, t0, L, 1, dev["k"], dev["v"], sel)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("L", [64, 1])
def test_rope_far_position(orc, L):
    """A chunk near position 300K: shifts of ~3e5 positions, where an fp32
    angle would be off by far more than the tolerance."""
    n_ctx, t0, d = 300_000, 299_900, 128
    w = LL.replace(n_ctx=n_ctx, batch=1, n_q_heads=4, n_kv_heads=1, window=512, top_k=8, chunk=L)
    g = torch.Generator().manual_seed(7)
    k = torch.randn((1, 1, n_ctx, d), generator=g).to(torch.bfloat16)
    v = torch.randn((1, 1, n_ctx, d), generator=g).to(torch.bfloat16)
    q = torch.randn((1, 4, L, d), generator=g).to(torch.bfloat16)
    sel = selections(orc, w, [t0], L, 4)
    theta = 500000.0
    cfg = cfg_of(w, rope_theta=theta)
    out, lse = gpu_attend(cfg, q.cuda(), 0, t0, L, 1, k.cuda(), v.cuda(),
                          torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attend_all(q, t0, k, v, sel[:, :, 0], B=w.block, n_init=w.n_init,
                                  W=w.window, rope_theta=theta)
    tol = tolerance(torch.bfloat16, o_ref)
    assert_close(out, o_ref, tol, "far out")
    err = np.abs(lse.cpu().numpy().astype(np.float64) - l_ref)
    l_tol = 1e-3
    if L >= 16:   # MFMA chunk path
        l_tol = l_tol + mfma_rounding_bound(w, q, k, t0, L)
    assert (err <= l_tol).all(), float(err.max())



def test_rope_varlen(orc, data):
    """Per-sequence positions: row b equals the single-position call at
    pos[b], bit for bit, and the oracle."""
    w, theta, inp, dev = data("bf16_g4")
    w2 = w.replace(batch=2)
    inp = synth.make_inputs(w2)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    cfg = cfg_of(w2, rope_theta=theta)
    L = 1
    pos_h = [w.n_ctx - 3, w.n_init // 2]
    sels = [selections(orc, w2, [p], L, 10 + p) for p in pos_h]
    sel = np.concatenate([sels[0][:1], sels[1][1:]], axis=0)
    sel_d = torch.from_numpy(sel).cuda()
    out = torch.empty((2, w.n_q_heads, 1, w.head_dim), dtype=q.dtype, device="cuda")
    lse = torch.empty((2, w.n_q_heads, 1), dtype=torch.float32, device="cuda")
    ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, 2, 0, L, 1)
    pos = torch.tensor(pos_h, dtype=torch.int64, device="cuda")
    # q row b sits at pos[b]: hand over the rows of each sequence's position
    qv = torch.stack([q[b, :, pos_h[b]] for b in range(2)])[:, :, None].contiguous()
    F.infllm_attend_varlen(cfg, qv, 0, pos, L, 1, k, v, sel_d, out, lse, ws=ws)
    torch.cuda.synchronize()
    for b in range(2):
        o1, l1 = gpu_attend(cfg, qv[b:b + 1], 0, pos_h[b], L, 1, k[b:b + 1], v[b:b + 1],
                            sel_d[b:b + 1].clone())   # sel rows must be 16-byte aligned
        torch.cuda.synchronize()
        assert torch.equal(out[b:b + 1], o1) and torch.equal(lse[b:b + 1], l1), b
        o_ref, l_ref = orc.attend_all(qv[b:b + 1].cpu(), pos_h[b], inp["k"][b:b + 1],
                                      inp["v"][b:b + 1], sel[b:b + 1, :, 0], B=w.block,
                                      n_init=w.n_init, W=w.window, rope_theta=theta)
        assert_close(out[b:b + 1], o_ref, tolerance(torch.bfloat16, o_ref), "varlen %d" % b)


@pytest.mark.parametrize("name,one_launch", [("bf16_g4", True), ("bf16_g8_ragged", False)])
def test_rope_select_attend(orc, data, name, one_launch):
    """The decode step with rope_theta set: in one launch where it fits
    (bf16, head_dim 128, up to 4 query heads a KV head), else the selection
    and attention calls.  Its selection and scores equal infllm_select_units
    bit for bit; its output equals the attention of that selection (bit for
    bit for the two calls, up to fp32 rounding in one launch, which splits
    the attention differently) and the oracle's; two calls on one workspace
    give the same bits."""
    w, theta, inp, dev = data(name)
    cfg = cfg_of(w, rope_theta=theta)
    plan = F.infllm_step_plan(cfg, w.batch, orc.num_units(w.n_ctx, w.block, w.n_init), 4)
    assert plan["fused"] == int(one_launch)
    n_pos, t0 = 4, w.n_ctx - 4
    U = orc.num_units(w.n_ctx, w.block, w.n_init)
    _, repr_o, _ = orc.build_units_all(inp["q"], inp["k"], w.n_ctx, B=w.block, n_init=w.n_init,
                                       W=w.window, r_k=w.rep_k, mode=w.rep_mode)
    repr_d = torch.from_numpy(repr_o.astype(np.float32)).cuda()
    ws = F.workspace(cfg, F.INFLLM_CALL_SELECT_ATTEND, w.batch, U, 1, n_pos)
    runs = []
    for _ in range(2):
        scores = torch.empty((w.batch, w.n_kv_heads, n_pos, U), dtype=torch.float32,
                             device="cuda")
        sel = torch.empty((w.batch, w.n_kv_heads, n_pos, w.top_k), dtype=torch.int32,
                          device="cuda")
        out = torch.empty((w.batch, w.n_q_heads, n_pos, w.head_dim), dtype=torch.bfloat16,
                          device="cuda")
        lse = torch.empty((w.batch, w.n_q_heads, n_pos), dtype=torch.float32, device="cuda")
        F.infllm_select_attend(cfg, dev["q"], t0, t0, n_pos, repr_d, dev["k"], dev["v"], scores,
                               sel, out, lse, ws=ws)
        runs.append((scores, sel, out, lse))
    scores, sel, out, lse = runs[0]
    s2 = torch.empty_like(scores)
    sel2 = torch.empty_like(sel)
    F.infllm_select_units(cfg, dev["q"], t0, t0, 1, n_pos, repr_d, s2, sel2,
                          ws=F.workspace(cfg, F.INFLLM_CALL_SELECT, w.batch, U, 1, n_pos))
    o2, l2 = gpu_attend(cfg, dev["q"], t0, t0, 1, n_pos, dev["k"], dev["v"], sel2)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(runs[0], runs[1]))
    assert torch.equal(sel, sel2) and torch.equal(scores, s2)
    if one_launch:
        o2h = o2.float().cpu().numpy()
        assert_close(out, o2h, tolerance(torch.bfloat16, o2h), "one launch vs two calls")
        assert_close(lse, l2.cpu().numpy(), 1e-4, "lse, one launch vs two calls")
        assert F.infllm_workspace_status(ws) == 0
    else:
        assert torch.equal(out, o2) and torch.equal(lse, l2)
    sel_h = sel.cpu().numpy()
    check_chunks(orc, w, theta, inp, out, lse, sel_h, [t0 + i for i in range(n_pos)], 1,
                 "select_attend")
