"""Seeded synthetic workloads for InfLLM's context-memory attention step.

This module only describes workloads and draws their inputs.  It holds none
of the method's arithmetic (no unit table, no scoring, no selection, no
attention), so the HIP path and the fp64 oracle can both be fed from it
without sharing any computation.

Workload shapes follow the model geometries and context lengths the InfLLM
pages evaluate (Llama-3-8B and Mistral-7B heads, 32K to 1M tokens); the
values are synthetic, drawn with ``torch.Generator`` from fixed seeds.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_ctx: int              # context tokens (built into memory units)
    block: int              # memory-unit size B
    n_init: int             # initial (sink) tokens
    window: int             # local window W
    rep_k: int              # representative tokens per unit r_k
    top_k: int              # retrieved units per chunk k_m
    chunk: int              # query chunk for encoding; 0 = no encoding pass
    decode_steps: int       # single-token decode steps after the context
    rep_mode: str           # "tokens" | "mean"
    dtype: str              # "f32" | "bf16"
    kv_dist: str            # "normal" | "mixture"
    scale: float            # std of Q/K/V entries
    planted: str            # "none" | "mean_query_block" | "decode_dir"
    planted_block: int = -1  # for "mean_query_block": absolute block index
    planted_per_head: int = 0  # for "decode_dir": planted units per (seq, KV head)
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_cap(self) -> int:
        """K/V rows needed: the context plus one row per decode step."""
        return self.n_ctx + self.decode_steps

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_LLAMA = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, block=128, n_init=128, window=4096,
              rep_k=4, rep_mode="tokens", dtype="bf16", kv_dist="normal",
              scale=1.0 / math.sqrt(128.0), planted="none")

WORKLOADS: dict[str, Workload] = {
    # Tiny single layer, fp32, one planted unit on tokens 1024..1151.
    "tiny_f32": Workload(name="tiny_f32", batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64,
                         n_ctx=4096, block=128, n_init=64, window=512, rep_k=4, top_k=4,
                         chunk=256, decode_steps=0, rep_mode="tokens", dtype="f32",
                         kv_dist="normal", scale=1.0, planted="mean_query_block",
                         planted_block=8, seed=1),
    # Llama-3-8B-shaped layer, 32K chunked encoding.
    "llama3_8b_32k_encode": Workload(name="llama3_8b_32k_encode", batch=1, n_ctx=32768,
                                     top_k=16, chunk=512, decode_steps=0, seed=2, **_LLAMA),
    # Llama-3-8B-shaped layer, 128K context, 256 decode steps, batch 4.
    "llama3_8b_128k_decode": Workload(name="llama3_8b_128k_decode", batch=4, n_ctx=131072,
                                      top_k=32, chunk=0, decode_steps=256, seed=3, **_LLAMA),
    # Llama-3-8B-shaped layer, 1M context, 256 decode steps, batch 2,
    # 8 planted units per (sequence, KV head).
    "llama3_8b_1m_decode": Workload(name="llama3_8b_1m_decode", batch=2, n_ctx=1048576,
                                    top_k=32, chunk=0, decode_steps=256, seed=4,
                                    **{**_LLAMA, "planted": "decode_dir"}, planted_per_head=8),
    # Mistral-7B-shaped layer, 64K, clustered keys, encoding then decode;
    # run with representative tokens and with the mean of keys.
    "mistral_7b_64k_tokens": Workload(name="mistral_7b_64k_tokens", batch=1, n_ctx=65536,
                                      top_k=32, chunk=512, decode_steps=256, seed=5,
                                      **{**_LLAMA, "kv_dist": "mixture"}),
    "mistral_7b_64k_mean": Workload(name="mistral_7b_64k_mean", batch=1, n_ctx=65536,
                                    top_k=32, chunk=512, decode_steps=256, seed=5,
                                    **{**_LLAMA, "kv_dist": "mixture", "rep_mode": "mean"}),
}

N_MIXTURE = 64          # mixture components for clustered keys / values
MIXTURE_NOISE = 0.05    # within-component std, in units of `scale`
PLANT_GAIN = 3.0        # planted keys: PLANT_GAIN * unit direction + noise
PLANT_NOISE = 0.1       # planted-key noise std, in units of `scale`


def _normal(shape, gen, device, std) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def _mixture(n: int, d: int, gen, device, std) -> torch.Tensor:
    """Rows drawn from a N_MIXTURE-component Gaussian mixture: component means
    ~ N(0, std^2 I), uniform assignment, within-component std MIXTURE_NOISE*std."""
    means = _normal((N_MIXTURE, d), gen, device, std)
    z = torch.randint(0, N_MIXTURE, (n,), generator=gen, device=device)
    return means[z] + _normal((n, d), gen, device, MIXTURE_NOISE * std)


def make_inputs(w: Workload, device: str | torch.device = "cpu") -> dict:
    """Draw one workload's tensors on `device`.

    q      [b, H_q, n_ctx, d]           queries of the context positions
    k, v   [b, H_kv, n_ctx + steps, d]  keys / values, row = absolute position
    q_dec  [b, H_q, steps, d]           decode queries (positions n_ctx + s)
    planted_units: LongTensor [b, H_kv, n] of planted unit blocks (or None)
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    dt = w.torch_dtype
    b, Hq, Hkv, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    n, cap, S = w.n_ctx, w.n_cap, w.decode_steps

    q = torch.empty((b, Hq, n, d), dtype=dt, device=dev)
    k = torch.empty((b, Hkv, cap, d), dtype=dt, device=dev)
    v = torch.empty((b, Hkv, cap, d), dtype=dt, device=dev)
    q_dec = torch.empty((b, Hq, S, d), dtype=dt, device=dev) if S > 0 else None
    # one (sequence, head) slice at a time keeps fp32 temporaries small
    for bi in range(b):
        for h in range(Hq):
            q[bi, h] = _normal((n, d), gen, dev, w.scale).to(dt)
            if S > 0:
                q_dec[bi, h] = _normal((S, d), gen, dev, w.scale).to(dt)
        for h in range(Hkv):
            if w.kv_dist == "mixture":
                k[bi, h] = _mixture(cap, d, gen, dev, w.scale).to(dt)
                v[bi, h] = _mixture(cap, d, gen, dev, w.scale).to(dt)
            else:
                k[bi, h] = _normal((cap, d), gen, dev, w.scale).to(dt)
                v[bi, h] = _normal((cap, d), gen, dev, w.scale).to(dt)

    planted = None
    B = w.block
    if w.planted == "mean_query_block":
        # keys of one block = PLANT_GAIN * (unit mean-query direction) + noise
        planted = torch.full((b, Hkv, 1), w.planted_block, dtype=torch.long)
        lo, hi = w.planted_block * B, (w.planted_block + 1) * B
        for bi in range(b):
            for h in range(Hkv):
                qm = q[bi, h * w.group:(h + 1) * w.group].float().sum(0).mean(0)
                qhat = qm / qm.norm()
                k[bi, h, lo:hi] = (PLANT_GAIN * qhat
                                   + _normal((hi - lo, d), gen, dev, PLANT_NOISE)).to(dt)
    elif w.planted == "decode_dir":
        # n distinct blocks per (sequence, KV head), drawn among blocks lying
        # wholly before the first decode step's window; their keys =
        # PLANT_GAIN * (unit direction of the group-summed decode queries'
        # mean) + noise
        first = -(-w.n_init // B)
        last = (n - w.window) // B - 1
        planted = torch.empty((b, Hkv, w.planted_per_head), dtype=torch.long)
        for bi in range(b):
            for h in range(Hkv):
                perm = torch.randperm(last - first, generator=gen, device=dev)[:w.planted_per_head]
                blocks = (perm + first).sort().values.cpu()
                planted[bi, h] = blocks
                qm = q_dec[bi, h * w.group:(h + 1) * w.group].float().sum(0).mean(0)
                qhat = qm / qm.norm()
                for j in blocks.tolist():
                    k[bi, h, j * B:(j + 1) * B] = (
                        PLANT_GAIN * qhat
                        + _normal((B, d), gen, dev, PLANT_NOISE * w.scale)).to(dt)
    return dict(q=q, k=k, v=v, q_dec=q_dec, planted_units=planted)


def make_layer_kv(w: Workload, layer: int, device: str | torch.device = "cpu"):
    """K and V [b, H_kv, n_ctx + steps, d] of another layer of the same
    workload: the same distribution, an independent seed per layer (no
    planted blocks).  Decode benchmarks rotate over several layers so that
    one step's K/V is not still cached from the previous step."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 1000 + layer)
    dt = w.torch_dtype
    b, Hkv, d, cap = w.batch, w.n_kv_heads, w.head_dim, w.n_cap
    k = torch.empty((b, Hkv, cap, d), dtype=dt, device=dev)
    v = torch.empty((b, Hkv, cap, d), dtype=dt, device=dev)
    for bi in range(b):
        for h in range(Hkv):
            if w.kv_dist == "mixture":
                k[bi, h] = _mixture(cap, d, gen, dev, w.scale).to(dt)
                v[bi, h] = _mixture(cap, d, gen, dev, w.scale).to(dt)
            else:
                k[bi, h] = _normal((cap, d), gen, dev, w.scale).to(dt)
                v[bi, h] = _normal((cap, d), gen, dev, w.scale).to(dt)
    return k, v


def stream_lengths(w: Workload) -> list[int]:
    """Context lengths of the sequences of a streaming (serving) run: the
    workload's context for sequence 0, then ragged shorter ones (each a
    different distance from a unit boundary)."""
    return [w.n_ctx - bi * (w.n_ctx // 16 + 37) for bi in range(w.batch)]


def make_stream_queries(w: Workload, q: torch.Tensor) -> torch.Tensor:
    """Queries of every position 0 .. n_cap-1 [b, H_q, n_cap, d]: the
    context's rows of q, then fresh rows (seeded) for the decode positions,
    which a streaming unit build reads when a unit leaves the window."""
    dev = q.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 1000 + 999)
    b, Hq, n, d = q.shape
    out = torch.empty((b, Hq, w.n_cap, d), dtype=q.dtype, device=dev)
    out[:, :, :n] = q
    if w.n_cap > n:
        for bi in range(b):
            out[bi, :, n:] = _normal((Hq, w.n_cap - n, d), gen, dev, w.scale).to(q.dtype)
    return out


def plant_dominant_block(k: torch.Tensor, block: int, B: int, direction: torch.Tensor,
                         margin: float = 1.5) -> None:
    """Overwrite every key of absolute block `block` (all sequences and heads
    of k [b, H_kv, n, d]) with c * direction/|direction|, c = margin * the
    largest key norm elsewhere -- a block whose keys all point along
    `direction` [b, H_kv, d] and are longer than any other key."""
    kmax = k.float().norm(dim=-1).amax(dim=-1, keepdim=True)          # [b, H_kv, 1]
    unit = direction.float() / direction.float().norm(dim=-1, keepdim=True)
    c = margin * kmax
    k[:, :, block * B:(block + 1) * B] = (c * unit).unsqueeze(2).to(k.dtype)
