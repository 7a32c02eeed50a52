"""Oracle on the synthetic workloads (CPU only): the tiny fp32 workload end
to end, and reduced versions of the large ones, checked with properties that
hold at any size."""
import numpy as np
import pytest
import torch

from block_level_kv_amd import synth


def encode_oracle(orc, w, inp):
    q, k, v = inp["q"], inp["k"], inp["v"]
    rep_idx, repr_, _ = orc.build_units_all(q, k, w.n_ctx, B=w.block, n_init=w.n_init,
                                            W=w.window, r_k=w.rep_k, mode=w.rep_mode)
    sels, outs = [], []
    for t0 in range(0, w.n_ctx, w.chunk):
        qc = q[:, :, t0:t0 + w.chunk]
        _, sel, e = orc.select_all(qc, t0, repr_, B=w.block, n_init=w.n_init, W=w.window,
                                   k_m=w.top_k)
        out, _ = orc.attend_all(qc, t0, k, v, sel, B=w.block, n_init=w.n_init, W=w.window)
        sels.append((t0, e, sel))
        outs.append(out)
    return rep_idx, repr_, sels, np.concatenate(outs, axis=2)


def test_tiny_workload_pipeline(orc):
    w = synth.WORKLOADS["tiny_f32"]
    inp = synth.make_inputs(w)
    rep_idx, repr_, sels, out = encode_oracle(orc, w, inp)
    U = orc.num_units(w.n_ctx, w.block, w.n_init)
    assert U == 32 and rep_idx.shape == (1, 1, 32, 4)
    # planted block 8 -> unit 8 (n_init 64 < B); its representatives lie in it
    pu = w.planted_block - w.n_init // w.block
    assert ((rep_idx[0, 0, pu] >= 1024) & (rep_idx[0, 0, pu] < 1152)).all()
    # recall of the planted unit over the chunks where it is eligible is a
    # reported quantity; it must be a fraction, and the unit is eligible in
    # the later chunks
    elig = [(t0, sel) for t0, e, sel in sels if e > pu]
    assert len(elig) == 16 - 6
    recall = np.mean([pu in sel[0, 0].tolist() for _, sel in elig])
    assert 0.0 <= recall <= 1.0
    assert np.isfinite(out).all()


def test_tiny_workload_all_units_is_dense(orc):
    w = synth.WORKLOADS["tiny_f32"].replace(n_ctx=1024, top_k=64, planted="none")
    inp = synth.make_inputs(w)
    _, _, _, out = encode_oracle(orc, w, inp)
    q, k, v = (inp[x][0, 0].double() for x in ("q", "k", "v"))
    logits = (q @ k.T) / np.sqrt(w.head_dim)
    mask = torch.ones(w.n_ctx, w.n_ctx, dtype=torch.bool).tril()
    want = torch.softmax(logits.masked_fill(~mask, -np.inf), -1) @ v
    np.testing.assert_allclose(out[0, 0], want.numpy(), atol=1e-11)


@pytest.mark.parametrize("name", ["llama3_8b_32k_encode", "mistral_7b_64k_tokens",
                                  "mistral_7b_64k_mean"])
def test_reduced_encode_workloads(orc, name):
    # same head geometry and hyper-parameters, shortened context and heads
    w = synth.WORKLOADS[name].replace(n_ctx=6144, n_q_heads=8, n_kv_heads=2)
    inp = synth.make_inputs(w)
    q = inp["q"]
    assert q.dtype == torch.bfloat16
    rep_idx, repr_, ks = orc.build_units_all(q, inp["k"], w.n_ctx, B=w.block, n_init=w.n_init,
                                             W=w.window, r_k=w.rep_k, mode=w.rep_mode)
    U = orc.num_units(w.n_ctx, w.block, w.n_init)
    assert repr_.shape == (1, 2, U, 128)
    t0 = w.n_ctx - w.chunk
    _, sel, e = orc.select_all(q[:, :, t0:], t0, repr_, B=w.block, n_init=w.n_init,
                               W=w.window, k_m=w.top_k)
    assert e == (t0 + w.chunk - 1 - w.window) // w.block
    assert ((sel >= 0).sum(-1) == min(e, w.top_k)).all()
    # every query of the chunk attends <= n_init + k_m*B + W keys
    for t in (t0, t0 + w.chunk - 1):
        n = orc.working_context(t, sel[0, 0], w.block, w.n_init, w.window).size
        assert n <= w.n_init + w.top_k * w.block + w.window


def test_decode_planting_recipe(orc):
    w = synth.WORKLOADS["llama3_8b_1m_decode"].replace(n_ctx=16384, batch=1, n_q_heads=4,
                                                       n_kv_heads=1, decode_steps=8,
                                                       planted_per_head=3)
    inp = synth.make_inputs(w)
    blocks = inp["planted_units"][0, 0].tolist()
    assert len(set(blocks)) == 3
    U = orc.num_units(w.n_ctx, w.block, w.n_init)
    e = orc.num_eligible(w.n_ctx, U, w.block, w.n_init, w.window)
    assert all(1 <= j and j - 1 < e for j in blocks)
    # planted keys are long and point the same way
    kp = inp["k"][0, 0, blocks[0] * 128:(blocks[0] + 1) * 128].float()
    assert kp.norm(dim=-1).min() > 2.5
