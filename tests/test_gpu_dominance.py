"""The "planted unit is always retrieved" property at a Llama-3-8B 128K
decode shape, through the HIP build, scoring and top-k (one sequence, 32/8
heads, d = 128, 1,023 units): a unit whose keys all point along a decode
query's group sum and are longer than any other key has the largest score
(Cauchy-Schwarz), so it is the top-1 of every KV head and in every
selection (the dominance construction of the oracle's pins, at full size;
InfLLM Guide, "Core Innovation 2", items 1-2)."""
import pytest
import torch

from block_level_kv_amd import infllm as F
from block_level_kv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["tokens", "mean"])
def test_dominant_unit_top1_at_128k(mode):
    w = synth.WORKLOADS["llama3_8b_128k_decode"].replace(batch=1)
    B, n_init, W, d = w.block, w.n_init, w.window, w.head_dim
    n_ctx, Hq, Hkv = w.n_ctx, w.n_q_heads, w.n_kv_heads
    G = Hq // Hkv
    g = torch.Generator(device="cuda").manual_seed(11)
    scale = d ** -0.5
    q = (torch.randn((1, Hq, n_ctx + 1, d), device="cuda", generator=g) * scale).to(torch.bfloat16)
    k = (torch.randn((1, Hkv, n_ctx + 1, d), device="cuda", generator=g) * scale).to(torch.bfloat16)
    t = n_ctx                                  # the first decode position
    qsum = q[:, :, t].double().reshape(1, Hkv, G, d).sum(2)        # [1, H_kv, d]
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B, n_init=n_init,
                        window=W, rep_k=w.rep_k, top_k=w.top_k,
                        rep_mode=F.INFLLM_REP_MEAN if mode == "mean" else F.INFLLM_REP_TOKENS)
    U = F.infllm_num_units(cfg, n_ctx)
    e = F.infllm_num_eligible(cfg, t, U)
    assert U == 1023 and e > 900
    for block in (n_init // B + 3, n_init // B + e // 2, n_init // B + e - 1):
        kk = k.clone()
        synth.plant_dominant_block(kk, block, B, qsum)
        repr_ = torch.empty((1, Hkv, U, d), dtype=torch.float32, device="cuda")
        rep = torch.empty((1, Hkv, U, w.rep_k), dtype=torch.int32, device="cuda") \
            if mode == "tokens" else None
        F.infllm_build_units(cfg, q, kk, n_ctx, rep, repr_,
                             F.workspace(cfg, F.INFLLM_CALL_BUILD, 1, n_ctx))
        scores = torch.empty((1, Hkv, 1, U), dtype=torch.float32, device="cuda")
        sel = torch.empty((1, Hkv, 1, w.top_k), dtype=torch.int32, device="cuda")
        F.infllm_select_units(cfg, q, t, t, 1, 1, repr_, scores, sel,
                              ws=F.workspace(cfg, F.INFLLM_CALL_SELECT, 1, U, 1, 1))
        torch.cuda.synchronize()
        u = block - n_init // B
        top1 = scores[0, :, 0, :e].argmax(dim=-1)
        assert (top1 == u).all(), (mode, block, top1.tolist())
        assert all(u in sel[0, h, 0].tolist() for h in range(Hkv)), (mode, block)
