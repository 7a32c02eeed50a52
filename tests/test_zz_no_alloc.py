"""infllm_select_attend_static (the decode step on the library's own scratch
memory, for callers that cannot allocate) against infllm_select_attend on a
caller workspace: the same scores, selections and outputs, bit for bit, on
consecutive calls of decreasing size (the scratch keeps the last call's
contents), in both the one-launch and the two-call form; and against the
oracle."""
import numpy as np
import pytest
import torch

from block_level_kv_amd import infllm as F
from gpu_helpers import assert_close, tolerance

pytestmark = pytest.mark.gpu


def _case(seed, b, Hq, Hkv, d, U, k_m, n_pos, W, n_init, dt):
    B = 128
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B, n_init=n_init,
                        window=W, rep_k=4, top_k=k_m,
                        dtype=F.INFLLM_BF16 if dt == "bf16" else F.INFLLM_F32)
    gen = torch.Generator().manual_seed(seed)
    t0 = (U + n_init // B) * B + W + 11          # every unit eligible at the last position
    cap = t0 + n_pos + 3
    scale = d ** -0.5
    q = (torch.randn((b, Hq, n_pos, d), generator=gen) * scale).to(dtype)
    k = (torch.randn((b, Hkv, cap, d), generator=gen) * scale).to(dtype)
    v = (torch.randn((b, Hkv, cap, d), generator=gen) * scale).to(dtype)
    repr_ = torch.randn((b, Hkv, U, d), generator=gen)
    return cfg, t0, q, k, v, repr_


def _outputs(cfg, q, repr_, n_pos):
    b, U = q.shape[0], repr_.shape[2]
    return (torch.full((b, cfg.n_kv_heads, n_pos, U), 3.0, dtype=torch.float32, device="cuda"),
            torch.full((b, cfg.n_kv_heads, n_pos, cfg.top_k), -7, dtype=torch.int32, device="cuda"),
            torch.zeros((b, cfg.n_q_heads, n_pos, cfg.head_dim), dtype=q.dtype, device="cuda"),
            torch.zeros((b, cfg.n_q_heads, n_pos), dtype=torch.float32, device="cuda"))


# (seed, batch, Hq, Hkv, d, units, k_m, positions, W, n_init, dtype, one launch)
CALLS = [
    (1, 2, 32, 8, 128, 600, 32, 2, 1024, 128, "bf16", True),
    (2, 1, 8, 2, 128, 150, 8, 1, 512, 128, "bf16", True),      # smaller: the second call
    (3, 1, 4, 1, 64, 40, 4, 1, 512, 64, "f32", False),         # the two-call form, smaller still
]


def test_static_scratch_matches_workspace_entry(orc):
    for seed, b, Hq, Hkv, d, U, k_m, n_pos, W, n_init, dt, fused in CALLS:
        print("case", seed, b, U, n_pos, dt, flush=True)
        cfg, t0, q, k, v, repr_ = _case(seed, b, Hq, Hkv, d, U, k_m, n_pos, W, n_init, dt)
        assert F.infllm_step_plan(cfg, b, U, n_pos)["fused"] == int(fused)
        qg, kg, vg, rg = q.cuda(), k.cuda(), v.cuda(), repr_.cuda()
        ws = F.workspace(cfg, F.INFLLM_CALL_SELECT_ATTEND, b, U, 1, n_pos)
        ref = _outputs(cfg, qg, rg, n_pos)
        F.infllm_select_attend(cfg, qg, 0, t0, n_pos, rg, kg, vg, *ref, ws=ws)
        got = _outputs(cfg, qg, rg, n_pos)
        F.infllm_select_attend_static(cfg, qg, 0, t0, n_pos, rg, kg, vg, *got)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x, y), "seed %d" % seed
        # the output against the oracle on the selection
        sel = got[1].cpu().numpy()
        for c in range(n_pos):
            o_ref, l_ref = orc.attend_all(q[:, :, c:c + 1], t0 + c, k, v, sel[:, :, c], B=128,
                                          n_init=n_init, W=W)
            assert_close(got[2][:, :, c:c + 1], o_ref, tolerance(q.dtype, o_ref),
                         "seed %d pos %d" % (seed, c))
            assert_close(got[3][:, :, c:c + 1], l_ref, 1e-3, "lse seed %d pos %d" % (seed, c))
