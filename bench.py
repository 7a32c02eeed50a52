"""Benchmark of InfLLM's context-memory attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload: a Llama-3-8B-shaped layer (32 query / 8 KV heads, head_dim
128, bf16), 32,768-token context, chunked encoding in 512-query chunks
processed one after another: one step = build the unit pool over the context
(representative tokens, r_k = 4), then for each chunk score every unit,
keep the top 16 per KV head and attend over 128 initial tokens + 16 units +
a 4,096-token window.  Decode workloads (--workload llama3_8b_128k_decode,
llama3_8b_1m_decode, mistral_7b_64k_*): the unit pool is built once
beforehand; one step = 256 consecutive single-token decode steps.

Prints ONE JSON line.  `value` is attended KV tokens per second over the
whole step (sum over sequences and query positions of the number of keys
each query attends).  `roofline` is for the attention kernel: algorithmic
work per launch (MFMA flops 4*d*H_q*sum|A(t)| for chunks; K/V + query +
output bytes for decode) divided by its average launch time, measured with
HIP events on the launch stream inside the timed region.  `cpu_baseline` is
the fp64 oracle on a bounded sample of the same work on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_level_kv_amd import infllm as F  # noqa: E402
from block_level_kv_amd import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def cfg_of(w: synth.Workload) -> F.infllm_config:
    return F.make_config(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                         block=w.block, n_init=w.n_init, window=w.window, rep_k=w.rep_k,
                         top_k=w.top_k,
                         rep_mode=F.INFLLM_REP_MEAN if w.rep_mode == "mean" else F.INFLLM_REP_TOKENS,
                         dtype=F.INFLLM_F32 if w.dtype == "f32" else F.INFLLM_BF16)


def attended_counts(w: synth.Workload, t0: int, L: int, sel: np.ndarray) -> np.ndarray:
    """|A(t)| for t = t0..t0+L-1 and every (sequence, KV head): sinks + the
    selected units' keys at least W behind t + the window.  sel [b, H_kv, k_m]."""
    t = np.arange(t0, t0 + L, dtype=np.int64)
    n = np.minimum(w.n_init, t + 1)
    win_lo = np.maximum(w.n_init, t - w.window + 1)
    n = n + np.maximum(t + 1 - win_lo, 0)
    out = np.broadcast_to(n, sel.shape[:2] + (L,)).astype(np.int64).copy()
    j0 = w.n_init // w.block
    cap = t - w.window + 1
    for idx in np.ndindex(sel.shape[:2]):
        for u in sel[idx]:
            if u < 0:
                continue
            lo = max((u + j0) * w.block, w.n_init)
            hi = (u + j0 + 1) * w.block
            out[idx] += np.maximum(np.minimum(hi, cap) - lo, 0)
    return out


class Pipeline:
    """Buffers and call sequence of one workload on the GPU."""

    def __init__(self, w: synth.Workload, dev: str = "cuda"):
        self.w, self.cfg, self.dev = w, cfg_of(w), dev
        t = time.time()
        self.inp = synth.make_inputs(w, device=dev)
        torch.cuda.synchronize()
        self.gen_s = time.time() - t
        b, Hkv, d = w.batch, w.n_kv_heads, w.head_dim
        self.U = F.infllm_num_units(self.cfg, w.n_ctx)
        self.repr = torch.empty((b, Hkv, self.U, d), dtype=torch.float32, device=dev)
        self.rep_idx = (torch.empty((b, Hkv, self.U, w.rep_k), dtype=torch.int32, device=dev)
                        if w.rep_mode == "tokens" else None)
        self.build_ws = F.workspace(self.cfg, F.INFLLM_CALL_BUILD, b, w.n_ctx, device=dev)
        self.scores = torch.empty((b, Hkv, 1, self.U), dtype=torch.float32, device=dev)
        L = w.chunk if (w.chunk > 0 and w.decode_steps == 0) else 1
        self.score_ws = F.workspace(self.cfg, F.INFLLM_CALL_SCORE, b, 0, L, 1, device=dev)
        self.sel = torch.empty((b, Hkv, 1, w.top_k), dtype=torch.int32, device=dev)
        self.encode = w.chunk > 0 and w.decode_steps == 0
        if self.encode:
            self.n_chunks = w.n_ctx // w.chunk
            self.out = torch.empty_like(self.inp["q"])
            self.attn_ws = F.workspace(self.cfg, F.INFLLM_CALL_ATTEND, b, 0, w.chunk, 1, device=dev)
            self.sel_log = torch.empty((self.n_chunks, b, Hkv, w.top_k), dtype=torch.int32,
                                       device=dev)
        else:
            self.out = torch.empty_like(self.inp["q_dec"])
            self.attn_ws = F.workspace(self.cfg, F.INFLLM_CALL_ATTEND, b, 0, 1, 1, device=dev)
            self.sel_log = torch.empty((w.decode_steps, b, Hkv, w.top_k), dtype=torch.int32,
                                       device=dev)

    def build(self):
        w = self.w
        F.infllm_build_units(self.cfg, self.inp["q"], self.inp["k"], w.n_ctx, self.rep_idx,
                             self.repr, self.build_ws)

    def step(self, events=None):
        """One pass of the hot path; `events` collects (start, end) pairs
        around each attention call."""
        w, cfg, inp = self.w, self.cfg, self.inp
        if self.encode:
            self.build()
            q, L, items = inp["q"], w.chunk, [(c, c * w.chunk, c * w.chunk)
                                               for c in range(self.n_chunks)]
        else:
            q, L, items = inp["q_dec"], 1, [(s, s, w.n_ctx + s) for s in range(w.decode_steps)]
        for i, q_off, pos in items:
            F.infllm_score_units(cfg, q, q_off, pos, L, 1, self.repr, self.scores, self.score_ws)
            sel = self.sel_log[i].unsqueeze(2)
            F.infllm_topk_units(cfg, self.scores, sel)
            if events is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            F.infllm_attend(cfg, q, q_off, pos, L, 1, inp["k"], inp["v"], sel, self.out, None,
                            q_off, self.attn_ws)
            if events is not None:
                e1.record()
                events.append((e0, e1))

    def work(self):
        """(attended KV tokens, attention flops, attention bytes) of one step."""
        w = self.w
        sel = self.sel_log.cpu().numpy()
        tokens = flops = 0
        nbytes = 0
        esz = 2 if w.dtype == "bf16" else 4
        for i in range(sel.shape[0]):
            t0, L = (i * w.chunk, w.chunk) if self.encode else (w.n_ctx + i, 1)
            cnt = attended_counts(w, t0, L, sel[i])                 # [b, H_kv, L]
            tokens += int(cnt.sum()) // w.n_kv_heads                # mean over KV heads
            flops += 4 * w.head_dim * w.group * int(cnt.sum())
            nbytes += int(cnt.sum()) * 2 * w.head_dim * esz         # K and V rows read
            nbytes += 2 * w.batch * w.n_q_heads * L * w.head_dim * esz  # q in, out
        return tokens, flops, nbytes


def cpu_baseline(w: synth.Workload, pipe: Pipeline) -> dict:
    """The oracle on a bounded sample: for chunked encoding, one chunk's score,
    top-k and attention plus that chunk's share of the unit build; for
    decode, two decode steps.  Value in attended KV tokens per second."""
    from oracle import oracle as orc
    inp = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in pipe.inp.items()}
    B, n_init, W = w.block, w.n_init, w.window
    G = w.group
    t_start = time.time()
    tokens = 0
    if pipe.encode:
        n_chunks = w.n_ctx // w.chunk
        U = orc.num_units(w.n_ctx, B, n_init)
        share = max(1, math.ceil(U / n_chunks))          # units per chunk of the build
        for h in range(w.n_kv_heads):
            if w.rep_mode == "mean":
                orc.build_mean(inp["k"][0, h], B, n_init, 0, share)
            else:
                orc.build_tokens(inp["q"][0, h * G:(h + 1) * G], inp["k"][0, h], w.n_ctx, B,
                                 n_init, W, w.rep_k, 0, share)
        repr_ = pipe.repr.cpu().double().numpy()
        t0 = w.n_ctx - w.chunk
        qc = inp["q"][:1, :, t0:]
        _, sel, _ = orc.select_all(qc, t0, repr_[:1], B=B, n_init=n_init, W=W, k_m=w.top_k)
        orc.attend_all(qc, t0, inp["k"][:1], inp["v"][:1], sel, B=B, n_init=n_init, W=W)
        tokens = int(attended_counts(w, t0, w.chunk, sel)[0, 0].sum())
        sample = ("1 of %d chunks (512 queries x %d heads, sequence 0) plus that chunk's share "
                  "(%d units x %d KV heads) of the unit build" % (n_chunks, w.n_q_heads, share,
                                                                   w.n_kv_heads))
    else:
        repr_ = pipe.repr.cpu().double().numpy()
        for s in range(2):
            t = w.n_ctx + s
            qd = inp["q_dec"][:1, :, s:s + 1]
            _, sel, _ = orc.select_all(qd, t, repr_[:1], B=B, n_init=n_init, W=W, k_m=w.top_k)
            orc.attend_all(qd, t, inp["k"][:1], inp["v"][:1], sel, B=B, n_init=n_init, W=W)
            tokens += int(attended_counts(w, t, 1, sel)[0, 0].sum())
        sample = "2 of %d decode steps, sequence 0 of %d" % (w.decode_steps, w.batch)
    dt = time.time() - t_start
    return {"value": tokens / dt, "unit": "attended KV tokens/s", "cores": orc.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_8b_32k_encode", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path runs on a single MI355X with the whole unit "
              "pool resident; runs on %d GPUs are not part of this benchmark" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    pipe = Pipeline(w)
    if not pipe.encode:
        pipe.build()
    for _ in range(args.warmup):
        pipe.step()
    torch.cuda.synchronize()

    events = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        pipe.step(events)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))

    tokens, flops, nbytes = pipe.work()
    n_calls = len(events) // args.steps
    if pipe.encode:
        achieved = flops / n_calls / (attn_ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None}
    else:
        achieved = nbytes / n_calls / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof["kernel"] = "infllm_attend"
    roof["avg_launch_us"] = round(attn_ms * 1e3, 2)
    roof["launches_per_step"] = n_calls

    line = {
        "metric": "attended KV tokens/s (InfLLM attention step, Llama-3-8B layer)",
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "attended KV tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_ctx": w.n_ctx,
                   "heads": "%dq/%dkv" % (w.n_q_heads, w.n_kv_heads), "head_dim": w.head_dim,
                   "chunk": w.chunk, "decode_steps": w.decode_steps, "block": w.block,
                   "n_init": w.n_init, "window": w.window, "rep_k": w.rep_k, "top_k": w.top_k,
                   "rep_mode": w.rep_mode, "attended_tokens_per_step": tokens},
        "roofline": roof,
    }
    if not pipe.encode:
        line["ms_per_decode_step"] = round(ms_step / w.decode_steps, 5)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, pipe)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
