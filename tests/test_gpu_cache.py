"""GPU unit cache over host-resident units (InfLLM Guide, "Core Innovation
3"): a run of decode steps through infllm_cache_fetch and
infllm_attend_cached, checked step by step against
  - the cache oracle (oracle/unit_cache.py): the slot, unit and stamp
    tables of every (sequence, KV head), and the hit / miss totals, exactly;
  - the host pool: every cached slot holds its unit's K/V block, bit for bit;
  - infllm_attend over the full resident K/V with the same selection: the
    output and LSE bit for bit (the same kernel arithmetic, keys from the
    slabs and the ring instead), and the attention oracle once.
Selections keep part of the previous step's units (locality) and bring new
ones, with empty slots and repeats, so the run has hits, misses and
evictions; the local keys come from a ring shorter than the context."""
import numpy as np
import pytest
import torch

from block_level_kv_amd import infllm as F
from gpu_helpers import assert_close, gpu_attend, tolerance
from oracle.unit_cache import UnitCache

pytestmark = pytest.mark.gpu


def parse_state(state, rows, U, C):
    """(hits, misses, slot_of [rows, U], unit_of [rows, C], stamp [rows, C]) with
    the stored +1 offsets removed (-1 = absent / empty)."""
    r = lambda x: (x + 255) // 256 * 256
    raw = state.cpu()
    hits, misses = raw[:16].view(torch.int64).tolist()
    o = 256
    slot_of = raw[o:o + rows * U * 4].view(torch.int32).reshape(rows, U) - 1
    o += r(rows * U * 4)
    unit_of = raw[o:o + rows * C * 4].view(torch.int32).reshape(rows, C) - 1
    o += r(rows * C * 4)
    stamp = raw[o:o + rows * C * 8].view(torch.int64).reshape(rows, C)
    return hits, misses, slot_of.numpy(), unit_of.numpy(), stamp.numpy()


def fill_ring(k_full, v_full, local_cap, n_init, t_max):
    """The local buffers of a call whose newest position is t_max: rows 0 ..
    n_init-1 the initial tokens, position p >= n_init at row n_init + (p -
    n_init) mod R for the R positions up to t_max."""
    R = local_cap - n_init
    kl = torch.zeros(k_full.shape[:2] + (local_cap, k_full.shape[3]), dtype=k_full.dtype,
                     device=k_full.device)
    vl = torch.zeros_like(kl)
    kl[:, :, :n_init] = k_full[:, :, :n_init]
    vl[:, :, :n_init] = v_full[:, :, :n_init]
    p = torch.arange(max(n_init, t_max - R + 1), t_max + 1, device=k_full.device)
    rows = n_init + (p - n_init) % R
    kl[:, :, rows] = k_full[:, :, p]
    vl[:, :, rows] = v_full[:, :, p]
    return kl, vl


@pytest.mark.parametrize("dt,Hq,Hkv,d,C,n_pos,n_init", [
    ("bf16", 8, 2, 128, 24, 1, 128),
    ("bf16", 16, 2, 128, 40, 2, 100),      # G = 8, two positions a call, sinks not B-aligned
    ("f32", 4, 4, 64, 16, 1, 64),          # fp32, d = 64, G = 1
])
def test_cache_steps(orc, dt, Hq, Hkv, d, C, n_pos, n_init):
    b, B, W, k_m, U = 2, 128, 512, 8, 90
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B, n_init=n_init,
                        window=W, rep_k=4, top_k=k_m,
                        dtype=F.INFLLM_BF16 if dt == "bf16" else F.INFLLM_F32)
    n_steps = 24
    t0 = (U + n_init // B) * B + W + 3          # every unit eligible from the first step
    ctx_cap = t0 + n_steps * n_pos + 8
    g = torch.Generator(device="cuda").manual_seed(21 + C)
    k_full = torch.randn((b, Hkv, ctx_cap, d), device="cuda", generator=g).to(dtype)
    v_full = torch.randn((b, Hkv, ctx_cap, d), device="cuda", generator=g).to(dtype)
    q_all = torch.randn((b, Hq, n_steps * n_pos, d), device="cuda", generator=g).to(dtype)
    k_host = torch.empty(k_full.shape, dtype=dtype, pin_memory=True)
    v_host = torch.empty(v_full.shape, dtype=dtype, pin_memory=True)
    k_host.copy_(k_full)
    v_host.copy_(v_full)
    cache_k = torch.zeros((b, Hkv, C, B, d), dtype=dtype, device="cuda")
    cache_v = torch.zeros_like(cache_k)
    state = F.cache_state(cfg, b, U, C)
    local_cap = n_init + W + n_pos - 1 + 37      # a ring that wraps during the run
    ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, 1, n_pos)
    rows = b * Hkv
    orc_caches = [UnitCache(C, U) for _ in range(rows)]
    rng = np.random.default_rng(C)
    prev = [rng.choice(U, size=k_m, replace=False) for _ in range(rows * n_pos)]
    hits_o = misses_o = 0
    for step in range(1, n_steps + 1):
        t = t0 + (step - 1) * n_pos
        # selection: half of the previous step's units, the rest new; an
        # empty slot and a repeat in each row
        sel = np.full((b, Hkv, n_pos, k_m), -1, np.int32)
        for r in range(rows * n_pos):
            keep = rng.choice(prev[r], size=k_m // 2, replace=False)
            new = rng.choice(np.setdiff1d(np.arange(U), keep), size=k_m - k_m // 2 - 2,
                             replace=False)
            ids = np.concatenate([keep, new, [keep[0]]]).astype(np.int32)
            rng.shuffle(ids)
            sel[r // (Hkv * n_pos), (r // n_pos) % Hkv, r % n_pos, :len(ids)] = ids
            prev[r] = np.concatenate([keep, new])
        sel_d = torch.from_numpy(sel).cuda()
        F.infllm_cache_fetch(cfg, sel_d, U, step, k_host, v_host, cache_k, cache_v, state)
        for r in range(rows):
            h_, m_, _ = orc_caches[r].fetch(step, sel[r // Hkv, r % Hkv].ravel())
            hits_o += h_
            misses_o += m_
        hits, misses, slot_of, unit_of, stamp = parse_state(state, rows, U, C)
        assert (hits, misses) == (hits_o, misses_o), step
        for r in range(rows):
            oc = orc_caches[r]
            assert unit_of[r].tolist() == oc.unit_of, (step, r)
            assert stamp[r].tolist() == oc.stamp, (step, r)
            assert slot_of[r].tolist() == oc.slot_of, (step, r)
        # slabs hold their units' blocks
        for r in range(rows):
            bi, h = r // Hkv, r % Hkv
            for c, u in enumerate(unit_of[r].tolist()):
                if u >= 0:
                    j = u + n_init // B
                    assert torch.equal(cache_k[bi, h, c], k_full[bi, h, j * B:(j + 1) * B]), (step, r, c)
                    assert torch.equal(cache_v[bi, h, c], v_full[bi, h, j * B:(j + 1) * B])
        # attention over the cache = attention over the resident K/V
        kl, vl = fill_ring(k_full, v_full, local_cap, n_init, t + n_pos - 1)
        q = q_all[:, :, (step - 1) * n_pos:step * n_pos].contiguous()
        out = torch.empty((b, Hq, n_pos, d), dtype=dtype, device="cuda")
        lse = torch.empty((b, Hq, n_pos), dtype=torch.float32, device="cuda")
        F.infllm_attend_cached(cfg, q, 0, t, n_pos, kl, vl, ctx_cap, sel_d, U, cache_k, cache_v,
                               state, out, lse, ws=ws)
        o_res, l_res = gpu_attend(cfg, q, 0, t, 1, n_pos, k_full, v_full, sel_d)
        torch.cuda.synchronize()
        assert torch.equal(out, o_res) and torch.equal(lse, l_res), step
        if step == n_steps:
            o_ref, l_ref = orc.attend_all(q[:, :, :1].cpu(), t, k_full.cpu(), v_full.cpu(),
                                          sel[:, :, 0], B=B, n_init=n_init, W=W)
            assert_close(out[:, :, :1], o_ref, tolerance(dtype, o_ref), "cached out")
    assert hits_o > 0 and misses_o > rows * C      # hits, and evictions (more misses than slots)


def test_cache_absent_unit_gives_nan_rows():
    """A selected unit that was never fetched: that (sequence, KV head)'s rows
    are NaN, the others as the resident attention."""
    b, Hq, Hkv, d, B, n_init, W, k_m, U, C = 1, 8, 2, 128, 128, 128, 512, 4, 40, 8
    cfg = F.make_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, block=B, n_init=n_init,
                        window=W, rep_k=4, top_k=k_m)
    t = (U + 1) * B + W + 5
    ctx_cap = t + 4
    g = torch.Generator(device="cuda").manual_seed(3)
    k_full = torch.randn((b, Hkv, ctx_cap, d), device="cuda", generator=g).to(torch.bfloat16)
    v_full = torch.randn_like(k_full)
    q = torch.randn((b, Hq, 1, d), device="cuda", generator=g).to(torch.bfloat16)
    k_host = torch.empty(k_full.shape, dtype=torch.bfloat16, pin_memory=True)
    v_host = torch.empty(k_full.shape, dtype=torch.bfloat16, pin_memory=True)
    k_host.copy_(k_full)
    v_host.copy_(v_full)
    cache_k = torch.zeros((b, Hkv, C, B, d), dtype=torch.bfloat16, device="cuda")
    cache_v = torch.zeros_like(cache_k)
    state = F.cache_state(cfg, b, U, C)
    sel = torch.tensor([[[[1, 5, 9, -1]], [[2, 6, 10, -1]]]], dtype=torch.int32, device="cuda")
    F.infllm_cache_fetch(cfg, sel, U, 1, k_host, v_host, cache_k, cache_v, state)
    sel2 = sel.clone()
    sel2[0, 1, 0, 3] = 30          # head 1 now also selects unit 30, never fetched
    kl, vl = fill_ring(k_full, v_full, n_init + W + 8, n_init, t)
    out = torch.empty((b, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, Hq, 1), dtype=torch.float32, device="cuda")
    F.infllm_attend_cached(cfg, q, 0, t, 1, kl, vl, ctx_cap, sel2, U, cache_k, cache_v, state,
                           out, lse, ws=F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, 1, 1))
    o_res, l_res = gpu_attend(cfg, q, 0, t, 1, 1, k_full, v_full, sel2)
    torch.cuda.synchronize()
    G = Hq // Hkv
    assert torch.equal(out[:, :G], o_res[:, :G]) and torch.equal(lse[:, :G], l_res[:, :G])
    assert torch.isnan(out[:, G:].float()).all() and torch.isnan(lse[:, G:]).all()
