"""infllm_select_attend_static under HIP graph capture (the callers it is
for): a decode step captured once and replayed several times, with eager
work and synchronisation between the replays, gives the eager call's
scores, selections and outputs bit for bit each time -- in the one-launch
form and in the two-call form -- and the scratch array it shares with eager
calls is left ready for them."""
import pytest
import torch

from block_level_kv_amd import infllm as F

pytestmark = pytest.mark.gpu


def _case(seed, b, Hq, Hkv, d, U, k_m, n_pos, W, n_init, dt):
    B = 128
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B, n_init=n_init,
                        window=W, rep_k=4, top_k=k_m,
                        dtype=F.INFLLM_BF16 if dt == "bf16" else F.INFLLM_F32)
    gen = torch.Generator().manual_seed(seed)
    t0 = (U + n_init // B) * B + W + 11
    cap = t0 + n_pos + 3
    scale = d ** -0.5
    q = (torch.randn((b, Hq, n_pos, d), generator=gen) * scale).to(dtype).cuda()
    k = (torch.randn((b, Hkv, cap, d), generator=gen) * scale).to(dtype).cuda()
    v = (torch.randn((b, Hkv, cap, d), generator=gen) * scale).to(dtype).cuda()
    repr_ = torch.randn((b, Hkv, U, d), generator=gen).cuda()
    return cfg, t0, q, k, v, repr_


def _outputs(cfg, q, repr_, n_pos):
    b, U = q.shape[0], repr_.shape[2]
    return (torch.empty((b, cfg.n_kv_heads, n_pos, U), dtype=torch.float32, device="cuda"),
            torch.empty((b, cfg.n_kv_heads, n_pos, cfg.top_k), dtype=torch.int32, device="cuda"),
            torch.empty((b, cfg.n_q_heads, n_pos, cfg.head_dim), dtype=q.dtype, device="cuda"),
            torch.empty((b, cfg.n_q_heads, n_pos), dtype=torch.float32, device="cuda"))


# (seed, batch, Hq, Hkv, d, units, k_m, positions, W, n_init, dtype, one launch)
CASES = [
    (11, 2, 32, 8, 128, 600, 32, 2, 1024, 128, "bf16", True),
    (12, 1, 4, 1, 64, 40, 4, 1, 512, 64, "f32", False),
]


@pytest.mark.parametrize("case", CASES)
def test_static_step_graph_replays(case):
    seed, b, Hq, Hkv, d, U, k_m, n_pos, W, n_init, dt, fused = case
    cfg, t0, q, k, v, repr_ = _case(seed, b, Hq, Hkv, d, U, k_m, n_pos, W, n_init, dt)
    assert F.infllm_step_plan(cfg, b, U, n_pos)["fused"] == int(fused)
    print("case", seed, flush=True)
    ref = _outputs(cfg, q, repr_, n_pos)
    F.infllm_select_attend_static(cfg, q, 0, t0, n_pos, repr_, k, v, *ref)   # also the warm-up
    torch.cuda.synchronize()
    got = _outputs(cfg, q, repr_, n_pos)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        F.infllm_select_attend_static(cfg, q, 0, t0, n_pos, repr_, k, v, *got)
    torch.cuda.synchronize()
    other = _outputs(cfg, q, repr_, n_pos)
    for r in range(3):
        for x in got:          # stale values the replay must overwrite
            x.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y), "replay %d" % r
        # an eager call between replays, on the same scratch array
        F.infllm_select_attend_static(cfg, q, 0, t0 + 1, n_pos, repr_, k, v, *other)
        torch.cuda.synchronize()
    eager = _outputs(cfg, q, repr_, n_pos)
    F.infllm_select_attend_static(cfg, q, 0, t0 + 1, n_pos, repr_, k, v, *eager)
    torch.cuda.synchronize()
    for x, y in zip(other, eager):
        assert torch.equal(x, y)
