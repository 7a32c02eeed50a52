"""Benchmark of InfLLM's context-memory attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Headline workload: a Llama-3-8B-shaped layer (32 query / 8 KV heads,
head_dim 128, bf16), 32,768-token context, chunked encoding in 512-query
chunks: one step = build the unit pool over the context (representative
tokens, r_k = 4), then for every chunk score every unit and keep the top 16
per KV head, then for every chunk attend over 128 initial tokens + 16 units
+ a 4,096-token window.  Selection never depends on attention outputs, so
each of the three stages covers all 64 chunks in one call; the record also
times the same pass chunk by chunk (one call of each kind per chunk).

Without --workload the same line then carries a sub-record ("workloads")
for every other workload: the 128K and 1M decode layers (unit pools built
once beforehand; one step = 256 consecutive single-token decode steps,
rotating over 4 layers' K/V and unit pools as a model's layers follow one
another, so no step finds its K/V still in the 256 MB last-level cache;
--layers 1 gives the single-layer figure), the Mistral-7B 64K layer with
representative tokens and with mean-of-keys units (one step = build + 128
encoding chunks + 256 decode steps) and the tiny fp32 layer.  --workload
NAME measures one workload only.

Before the W warm-up steps, untimed steps run for --settle seconds (1 by
default) so that the GPU clocks are in steady state when timing starts.

Prints ONE JSON line.  `value` is attended KV tokens per second over the
whole step (over sequences and query positions, the number of keys each
query attends, averaged over KV heads).  `roofline` is for the attention
kernel of the dominant pass (chunked encoding if the workload has one):
algorithmic work per launch -- MFMA flops 4*d*H_q*sum|A(t)| for chunks, or
the K/V rows, queries, outputs (and unit rows, for the one-launch decode
step) it must move for decode -- divided by its average launch time: HIP
events on the launch stream, inside the timed region, around each step's
attention launches; `frac_from_profile` is the same work over the kernel's
average in the committed rocprofv3 trace.  `cpu_baseline` is the fp64
oracle on a bounded sample of the same work on the host cores.
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


def cfg_of(w: synth.Workload, rope_theta: float = 0.0) -> F.infllm_config:
    """The library configuration of a workload; rope_theta > 0: the attention
    re-positions q and k inside the working context (keys otherwise arrive
    turned at their absolute positions)."""
    return F.make_config(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                         block=w.block, n_init=w.n_init, window=w.window, rep_k=w.rep_k,
                         top_k=w.top_k,
                         rep_mode=F.INFLLM_REP_MEAN if w.rep_mode == "mean" else F.INFLLM_REP_TOKENS,
                         dtype=F.INFLLM_F32 if w.dtype == "f32" else F.INFLLM_BF16,
                         rope_theta=rope_theta)


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
    """Buffers and call sequence of one workload on the GPU.  The encoding
    pass (if w.chunk > 0) builds the unit pool and runs every chunk; the
    decode pass (if w.decode_steps > 0) runs single-token steps against the
    pool.  Selections and outputs of the last step are kept for checking."""

    def __init__(self, w: synth.Workload, dev: str = "cuda", layers: int = 1,
                 fused_step: bool = True, rope_theta: float = 0.0):
        self.w, self.cfg, self.dev = w, cfg_of(w, rope_theta), dev
        t = time.time()
        self.inp = synth.make_inputs(w, device=dev)
        torch.cuda.synchronize()
        self.gen_s = time.time() - t
        b, Hkv, d = w.batch, w.n_kv_heads, w.head_dim
        cfg = self.cfg
        self.encode = w.chunk > 0
        self.decode = w.decode_steps > 0
        self.U = F.infllm_num_units(cfg, w.n_ctx)
        self.repr = torch.empty((b, Hkv, self.U, d), dtype=torch.float32, device=dev)
        self.rep_idx = (torch.empty((b, Hkv, self.U, w.rep_k), dtype=torch.int32, device=dev)
                        if w.rep_mode == "tokens" else None)
        self.build_ws = F.workspace(cfg, F.INFLLM_CALL_BUILD, b, w.n_ctx, device=dev)
        self.scores = torch.empty((b, Hkv, 1, self.U), dtype=torch.float32, device=dev)
        # chunks of whole units take their query sums from the build's block
        # sums (infllm_build_units_qsum / infllm_score_units_qsum): the
        # encoding pass reads the queries for them once, in the build
        self.block_qsum = None
        if w.chunk > 0 and w.chunk % w.block == 0:
            nb = (w.n_ctx + w.block - 1) // w.block
            self.block_qsum = torch.empty((b, Hkv, nb, d), dtype=torch.float64, device=dev)
            self.build_ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_QSUM, b, w.n_ctx, device=dev)
        if self.encode:
            nc = self.n_chunks = w.n_ctx // w.chunk
            self.enc_scores = torch.empty((b, Hkv, nc, self.U), dtype=torch.float32, device=dev)
            self.enc_score_ws = F.workspace(cfg, F.INFLLM_CALL_SCORE, b, 0, w.chunk, nc, device=dev)
            self.enc_attn_ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, w.chunk, nc, device=dev)
            self.enc_sel = torch.empty((b, Hkv, nc, w.top_k), dtype=torch.int32, device=dev)
            # per-chunk view [chunk, b, H_kv, 1, k_m]
            self.sel_enc = self.enc_sel.permute(2, 0, 1, 3).unsqueeze(3)
            self.out_enc = torch.empty_like(self.inp["q"])
            # the chunk-by-chunk form's buffers (one chunk per call)
            self.seq_scores = torch.empty((b, Hkv, 1, self.U), dtype=torch.float32, device=dev)
            self.seq_sel = torch.empty((b, Hkv, 1, w.top_k), dtype=torch.int32, device=dev)
            self.seq_score_ws = F.workspace(cfg, F.INFLLM_CALL_SCORE, b, 0, w.chunk, 1, device=dev)
            self.seq_attn_ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, w.chunk, 1, device=dev)
        if self.decode:
            self.dec_score_ws = F.workspace(cfg, F.INFLLM_CALL_SELECT, b, 0, 1, 1, device=dev)
            self.dec_attn_ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, 1, 1, device=dev)
            self.sel_dec = torch.empty((w.decode_steps, b, Hkv, 1, w.top_k), dtype=torch.int32,
                                       device=dev)
            self.out_dec = torch.empty_like(self.inp["q_dec"])
        # a decode step in one launch (infllm_select_attend) where the
        # library's plan allows it
        self.fused = bool(fused_step and self.decode
                          and F.infllm_step_plan(cfg, b, self.U, 1)["fused"])
        if self.fused:
            self.dec_step_ws = F.workspace(cfg, F.INFLLM_CALL_SELECT_ATTEND, b, self.U, 1, 1,
                                           device=dev)
        # Layer 0 is the workload's own K/V; further layers (decode only)
        # have their own K/V, unit pool and selections, over the same queries
        self.layers = [dict(k=self.inp["k"], v=self.inp["v"], repr=self.repr,
                            rep_idx=self.rep_idx)]
        for li in range(1, layers):
            k, v = synth.make_layer_kv(w, li, device=dev)
            self.layers.append(dict(k=k, v=v, repr=torch.empty_like(self.repr),
                                    rep_idx=None if self.rep_idx is None
                                    else torch.empty_like(self.rep_idx)))
        torch.cuda.synchronize()

    def build(self, layer: int = 0):
        ly = self.layers[layer]
        if self.block_qsum is not None and layer == 0:
            F.infllm_build_units_qsum(self.cfg, self.inp["q"], ly["k"], self.w.n_ctx,
                                      ly["rep_idx"], ly["repr"], self.block_qsum, self.build_ws)
        else:
            F.infllm_build_units(self.cfg, self.inp["q"], ly["k"], self.w.n_ctx, ly["rep_idx"],
                                 ly["repr"], self.build_ws)

    def build_all(self):
        for li in range(len(self.layers)):
            self.build(li)

    def _select(self, q, q_off, pos, L, sel, score_ws, layer=0):
        # scores and top-k in one call (one launch for decode-sized chunks)
        F.infllm_select_units(self.cfg, q, q_off, pos, L, 1, self.layers[layer]["repr"],
                              self.scores, sel, ws=score_ws)

    def _attend(self, q, q_off, pos, L, sel, out, attn_ws, layer=0):
        ly = self.layers[layer]
        F.infllm_attend(self.cfg, q, q_off, pos, L, 1, ly["k"], ly["v"], sel, out, None, q_off,
                        attn_ws)

    @staticmethod
    def _mark(marks, key):
        if marks is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.setdefault(key, []).append(e)

    def step(self, marks=None):
        """One pass of the hot path.  Selection depends only on the built
        units, never on attention outputs, so each pass first scores and
        selects units for all of its query chunks (or decode positions) and
        then attends: the encoding pass with one call per kind covering all
        chunks, the decode pass one call per position (each decode step
        follows the previous one); where the fused decode step applies, one
        infllm_select_attend launch per position does both.  With a dict,
        events are recorded at the phase boundaries: 'enc_sel' / 'enc_end'
        around the encoding attention launch, 'dec_sel' / 'dec_end' around
        the decode attention (or fused step) launches."""
        w, inp, cfg = self.w, self.inp, self.cfg
        if self.encode:
            # the whole encoding pass: every chunk in one call of each kind
            # (chunk c covers queries [c*chunk, (c+1)*chunk), positions equal)
            self.build()
            nc = self.n_chunks
            if self.block_qsum is not None:
                F.infllm_score_units_qsum(cfg, self.block_qsum, 0, w.chunk, nc, self.repr,
                                          self.enc_scores)
            else:
                F.infllm_score_units(cfg, inp["q"], 0, 0, w.chunk, nc, self.repr, self.enc_scores,
                                     self.enc_score_ws)
            F.infllm_topk_units(cfg, self.enc_scores, self.enc_sel)
            self._mark(marks, "enc_sel")
            F.infllm_attend(cfg, inp["q"], 0, 0, w.chunk, nc, inp["k"], inp["v"], self.enc_sel,
                            self.out_enc, None, 0, self.enc_attn_ws)
            self._mark(marks, "enc_end")
        if self.decode and self.fused:
            # one launch per decode step: scores, selection and attention
            nl = len(self.layers)
            self._mark(marks, "dec_sel")
            for s in range(w.decode_steps):
                ly = self.layers[s % nl]
                F.infllm_select_attend(cfg, inp["q_dec"], s, w.n_ctx + s, 1, ly["repr"], ly["k"],
                                       ly["v"], self.scores, self.sel_dec[s], self.out_dec, None,
                                       s, ws=self.dec_step_ws)
            self._mark(marks, "dec_end")
        elif self.decode:
            # decode step s runs on layer s mod L, as a model's layers follow
            # one another
            nl = len(self.layers)
            for s in range(w.decode_steps):
                self._select(inp["q_dec"], s, w.n_ctx + s, 1, self.sel_dec[s], self.dec_score_ws,
                             s % nl)
            self._mark(marks, "dec_sel")
            for s in range(w.decode_steps):
                self._attend(inp["q_dec"], s, w.n_ctx + s, 1, self.sel_dec[s], self.out_dec,
                             self.dec_attn_ws, s % nl)
            self._mark(marks, "dec_end")

    def step_sequential(self):
        """The encoding pass with one call of each kind per chunk, chunk after
        chunk (the chunk-by-chunk form of the same work: the results are
        identical to step()'s)."""
        w, inp, cfg = self.w, self.inp, self.cfg
        self.build()
        for c in range(self.n_chunks):
            t0 = c * w.chunk
            if self.block_qsum is not None:
                F.infllm_score_units_qsum(cfg, self.block_qsum, t0, w.chunk, 1, self.repr,
                                          self.seq_scores)
            else:
                F.infllm_score_units(cfg, inp["q"], t0, t0, w.chunk, 1, self.repr, self.seq_scores,
                                     self.seq_score_ws)
            F.infllm_topk_units(cfg, self.seq_scores, self.seq_sel)
            F.infllm_attend(cfg, inp["q"], t0, t0, w.chunk, 1, inp["k"], inp["v"], self.seq_sel,
                            self.out_enc, None, t0, self.seq_attn_ws)

    def work(self):
        """Per pass: (attended KV tokens, attention flops, attention bytes)."""
        w = self.w
        esz = 2 if w.dtype == "bf16" else 4
        res = {}
        passes = []
        if self.encode:
            passes.append(("encode", self.sel_enc, [(c * w.chunk, w.chunk)
                                                    for c in range(self.n_chunks)]))
        if self.decode:
            passes.append(("decode", self.sel_dec, [(w.n_ctx + s, 1)
                                                    for s in range(w.decode_steps)]))
        for name, sel_log, items in passes:
            sel = sel_log.cpu().numpy()[:, :, :, 0]
            tokens = flops = nbytes = 0
            for i, (t0, L) in enumerate(items):
                cnt = attended_counts(w, t0, L, sel[i])             # [b, H_kv, L]
                tokens += int(cnt.sum()) // w.n_kv_heads             # mean over KV heads
                flops += 4 * w.head_dim * w.group * int(cnt.sum())
                nbytes += int(cnt.sum()) * 2 * w.head_dim * esz      # K and V rows read
                nbytes += 2 * w.batch * w.n_q_heads * L * w.head_dim * esz  # q in, out
                if name == "decode" and self.fused:
                    # the fused launch also reads every unit row and writes its score
                    nbytes += w.batch * w.n_kv_heads * self.U * (w.head_dim + 1) * 4
            res[name] = (tokens, flops, nbytes)
        return res


class StreamPipeline:
    """Serving-style decode with a growing unit pool (streaming unit build,
    variable-length batch).  The sequences of the batch have ragged context
    lengths (synth.stream_lengths) and decode at their own positions; each
    decode step is one selection and one attention call over the whole
    batch with a device array of per-sequence positions.  A unit joins a
    sequence's pool when its first key leaves that sequence's local window:
    it is built then (infllm_build_units_range, one call per sequence and
    layer that gains units) from the queries up to the current position.
    The pools of the starting contexts are built beforehand, each from its
    whole context.  Decode steps rotate over `layers` layers as in Pipeline;
    every layer's pool gains its units at the same step."""

    encode, decode = False, True

    def __init__(self, w: synth.Workload, dev: str = "cuda", layers: int = 1,
                 rope_theta: float = 0.0):
        self.w, self.cfg, self.dev = w, cfg_of(w, rope_theta), dev
        cfg = self.cfg
        self.inp = synth.make_inputs(w, device=dev)
        self.q_all = synth.make_stream_queries(w, self.inp["q"])
        self.lens = synth.stream_lengths(w)
        b, Hkv, d, S = w.batch, w.n_kv_heads, w.head_dim, w.decode_steps
        self.U = F.infllm_num_units(cfg, w.n_cap)              # pool rows
        self.scores = torch.empty((b, Hkv, 1, self.U), dtype=torch.float32, device=dev)
        self.sel_dec = torch.empty((S, b, Hkv, 1, w.top_k), dtype=torch.int32, device=dev)
        self.out_dec = torch.empty_like(self.inp["q_dec"])
        self.sel_ws = F.workspace(cfg, F.INFLLM_CALL_SELECT, b, 0, 1, 1, device=dev)
        self.attn_ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, 1, 1, device=dev)
        # one launch per decode step (infllm_select_attend) where it applies
        self.fused = bool(F.infllm_step_plan(cfg, b, self.U, 1)["fused"])
        if self.fused:
            self.step_ws = F.workspace(cfg, F.INFLLM_CALL_SELECT_ATTEND, b, self.U, 1, 1,
                                       device=dev)
        self.pos_host = np.array([[self.lens[bi] + s for bi in range(b)] for s in range(S)],
                                 dtype=np.int64)
        self.pos = torch.tensor(self.pos_host, dtype=torch.int64, device=dev)   # [S, b]
        tokens = w.rep_mode == "tokens"

        def pool():
            return dict(repr=torch.zeros((b, Hkv, self.U, d), dtype=torch.float32, device=dev),
                        rep_idx=(torch.full((b, Hkv, self.U, w.rep_k), -1, dtype=torch.int32,
                                            device=dev) if tokens else None))
        self.layers = [dict(k=self.inp["k"], v=self.inp["v"], **pool())]
        for li in range(1, layers):
            k, v = synth.make_layer_kv(w, li, device=dev)
            self.layers.append(dict(k=k, v=v, **pool()))
        self.repr = self.layers[0]["repr"]

        def elig(t):
            return F.infllm_num_eligible(cfg, t, self.U)
        # units each sequence holds before the first step, and the ranges it
        # gains at each step (built with the queries up to that position)
        self.start = [elig(n - 1) for n in self.lens]
        self.builds = []
        for s in range(S):
            todo = []
            for bi in range(b):
                t = int(self.pos_host[s, bi])
                lo, hi = elig(t - 1), elig(t)
                if hi > lo:
                    todo.append((bi, lo, hi, t + 1))
            self.builds.append(todo)
        self.n_builds = sum(len(x) for x in self.builds)
        most = max([hi - lo for todo in self.builds for _, lo, hi, _ in todo] + [1])
        self.range_ws = F.workspace(cfg, F.INFLLM_CALL_BUILD_RANGE, 1, most, device=dev)
        torch.cuda.synchronize()

    def _build(self, ly, bi, lo, hi, n, ws):
        sl = slice(bi, bi + 1)
        F.infllm_build_units_range(self.cfg, self.q_all[sl], ly["k"][sl], n, lo, hi,
                                   None if ly["rep_idx"] is None else ly["rep_idx"][sl],
                                   ly["repr"][sl], ws)

    def build_all(self):
        """The pools of the starting contexts (each sequence's own length)."""
        ws = F.workspace(self.cfg, F.INFLLM_CALL_BUILD_RANGE, 1, max(self.start + [1]),
                         device=self.dev)
        for ly in self.layers:
            for bi, n in enumerate(self.lens):
                if self.start[bi] > 0:
                    self._build(ly, bi, 0, self.start[bi], n, ws)

    @staticmethod
    def _mark(marks, key):
        Pipeline._mark(marks, key)

    def step(self, marks=None):
        """One pass of w.decode_steps steps: the units each step adds and its
        selection, in step order, then the attentions (selections never
        depend on attention outputs; a unit added at a later step is not
        eligible earlier).  Marks 'dec_sel' / 'dec_end' around the attention
        launches.  With the fused step: the units of every step, in step
        order, then one infllm_select_attend launch per step (marked); a
        unit built ahead of its step is not eligible before it, so the
        selections are the same."""
        w, cfg, q = self.w, self.cfg, self.inp["q_dec"]
        nl = len(self.layers)
        if self.fused:
            for s in range(w.decode_steps):
                for ly in self.layers:
                    for bi, lo, hi, n in self.builds[s]:
                        self._build(ly, bi, lo, hi, n, self.range_ws)
            self._mark(marks, "dec_sel")
            for s in range(w.decode_steps):
                ly = self.layers[s % nl]
                F.infllm_select_attend(cfg, q, s, 0, 1, ly["repr"], ly["k"], ly["v"], self.scores,
                                       self.sel_dec[s], self.out_dec, None, s, pos=self.pos[s],
                                       ws=self.step_ws)
            self._mark(marks, "dec_end")
            return
        for s in range(w.decode_steps):
            for ly in self.layers:
                for bi, lo, hi, n in self.builds[s]:
                    self._build(ly, bi, lo, hi, n, self.range_ws)
            F.infllm_select_units(cfg, q, s, 0, 1, 1, self.layers[s % nl]["repr"], self.scores,
                                  self.sel_dec[s], pos=self.pos[s], ws=self.sel_ws)
        self._mark(marks, "dec_sel")
        for s in range(w.decode_steps):
            ly = self.layers[s % nl]
            F.infllm_attend_varlen(cfg, q, s, self.pos[s], 1, 1, ly["k"], ly["v"], self.sel_dec[s],
                                   self.out_dec, None, s, self.attn_ws)
        self._mark(marks, "dec_end")

    def work(self):
        w = self.w
        esz = 2 if w.dtype == "bf16" else 4
        sel = self.sel_dec.cpu().numpy()[:, :, :, 0]
        tokens = flops = nbytes = 0
        for s in range(w.decode_steps):
            for bi in range(w.batch):
                cnt = attended_counts(w, int(self.pos_host[s, bi]), 1, sel[s, bi:bi + 1])
                tokens += int(cnt.sum()) // w.n_kv_heads
                flops += 4 * w.head_dim * w.group * int(cnt.sum())
                nbytes += int(cnt.sum()) * 2 * w.head_dim * esz
            nbytes += 2 * w.batch * w.n_q_heads * w.head_dim * esz
            if self.fused:   # every pool row read and scored
                nbytes += w.batch * w.n_kv_heads * self.U * (w.head_dim + 1) * 4
        return {"decode": (tokens, flops, nbytes)}


CPU_SAMPLE_SECONDS = 10.0


def cpu_baseline(w: synth.Workload, pipe: Pipeline, seconds: float = CPU_SAMPLE_SECONDS) -> dict:
    """The oracle on a bounded sample of the same work, about
    CPU_SAMPLE_SECONDS long: for chunked encoding, whole chunks (score, top-k,
    attention, sequence 0) from the last backwards, each with its share of
    the unit build; for decode, consecutive decode steps of sequence 0.
    Value in attended KV tokens per second."""
    from oracle import oracle as orc
    B, n_init, W = w.block, w.n_init, w.window
    G = w.group
    repr_ = pipe.repr.cpu().double().numpy()
    k0, v0 = pipe.inp["k"][:1].cpu(), pipe.inp["v"][:1].cpu()
    t_start = time.time()
    tokens = 0
    if pipe.encode:
        q0 = pipe.inp["q"][:1].cpu()
        n_chunks = w.n_ctx // w.chunk
        U = orc.num_units(w.n_ctx, B, n_init)
        share = max(1, math.ceil(U / n_chunks))          # units per chunk of the build
        done = 0
        while done < n_chunks and time.time() - t_start < seconds:
            u0 = min(done * share, max(U - share, 0))
            for h in range(w.n_kv_heads):
                if w.rep_mode == "mean":
                    orc.build_mean(k0[0, h], B, n_init, u0, min(u0 + share, U))
                else:
                    orc.build_tokens(q0[0, h * G:(h + 1) * G], k0[0, h], w.n_ctx, B, n_init, W,
                                     w.rep_k, u0, min(u0 + share, U))
            t0 = w.n_ctx - (done + 1) * w.chunk
            qc = q0[:, :, t0:t0 + w.chunk]
            _, sel, _ = orc.select_all(qc, t0, repr_[:1], B=B, n_init=n_init, W=W, k_m=w.top_k)
            orc.attend_all(qc, t0, k0, v0, sel, B=B, n_init=n_init, W=W)
            tokens += int(attended_counts(w, t0, w.chunk, sel).sum()) // w.n_kv_heads
            done += 1
        sample = ("%d of %d chunks (%d queries x %d heads each, sequence 0), each with its share "
                  "(%d units x %d KV heads) of the unit build" % (done, n_chunks, w.chunk,
                                                                   w.n_q_heads, share,
                                                                   w.n_kv_heads))
    else:
        qd0 = pipe.inp["q_dec"][:1].cpu()
        done = 0
        while done < w.decode_steps and time.time() - t_start < seconds:
            s = done
            t = w.n_ctx + s
            qd = qd0[:, :, s:s + 1]
            _, sel, _ = orc.select_all(qd, t, repr_[:1], B=B, n_init=n_init, W=W, k_m=w.top_k)
            orc.attend_all(qd, t, k0, v0, sel, B=B, n_init=n_init, W=W)
            tokens += int(attended_counts(w, t, 1, sel).sum()) // w.n_kv_heads
            done += 1
        sample = "%d of %d decode steps (score, top-k, attention), sequence 0 of %d" % (
            done, w.decode_steps, w.batch)
    dt = time.time() - t_start
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                       cpu)
    except OSError:
        pass
    return {"value": round(tokens / dt, 1), "unit": "attended KV tokens/s",
            "cores": orc.num_threads(), "kind": "oracle", "sample": sample,
            "seconds": round(dt, 2), "cpu": cpu, "host_cpus": os.cpu_count()}


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>.md), or None if there is none or the
    kernel's sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s_%s.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip()
    try:
        # one file, or a comma-separated list hashed in order
        h = hashlib.sha256()
        for src in fields["kernel_source"].split(","):
            h.update(open(os.path.join(ROOT, src.strip()), "rb").read())
        if h.hexdigest() != fields["kernel_source_sha256"]:
            return None
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def stored_profile_us(kernel: str, workload: str):
    """Average duration (us) of the kernel in the committed rocprofv3 kernel
    trace summary (profiles/<kernel>_<workload>.md: field avg_launch_us), or
    None if there is none or the kernel's sources have changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s_%s.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip()
    try:
        h = hashlib.sha256()
        for src in fields["kernel_source"].split(","):
            h.update(open(os.path.join(ROOT, src.strip()), "rb").read())
        if h.hexdigest() != fields["kernel_source_sha256"]:
            return None
        return float(fields["avg_launch_us"])
    except (KeyError, OSError, ValueError):
        return None


def measure_peaks() -> dict:
    """What plain library kernels reach on this GPU, as context for the
    published peaks: a 2 GiB device copy (bytes read + written) and a bf16
    8192^3 GEMM (hipBLASLt through torch.matmul).  Best of 5 runs each."""
    def best_ms(f, reps=5):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)
    x = torch.ones((1 << 29,), dtype=torch.float32, device="cuda")       # 2 GiB
    y = torch.empty_like(x)
    y.copy_(x)
    copy_ms = best_ms(lambda: y.copy_(x))                                 # 2 GiB in, 2 GiB out
    del x, y
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    torch.matmul(a, b)
    gemm_ms = best_ms(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": round((1 << 32) / (copy_ms * 1e-3) / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1)}


def roofline(w: synth.Workload, phase: str, work, attn_ms: float, n_calls: int,
             peaks: dict | None = None, fused: bool = False) -> dict:
    """attn_ms: average duration of one attention launch, in ms."""
    tokens, flops, nbytes = work
    if phase == "encode" and w.dtype == "bf16":
        achieved = flops / n_calls / (attn_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s"}
    elif phase == "encode":
        achieved = flops / n_calls / (attn_ms * 1e-3) / 1e12
        r = {"bound": "alu", "achieved": round(achieved, 2), "peak": PEAK_F32_TFLOPS,
             "unit": "TFLOP/s"}
    else:
        achieved = nbytes / n_calls / (attn_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    r["frac"] = round(achieved / r["peak"], 4)
    if peaks:   # the same work against what plain library kernels reach here
        if r["bound"] == "hbm":
            r["measured_peak"] = peaks["hbm_copy_GBs"]
            r["measured_peak_kernel"] = "2 GiB device copy, bytes read + written (torch copy_)"
        elif r["bound"] == "mfma":
            r["measured_peak"] = peaks["bf16_gemm_TFLOPs"]
            r["measured_peak_kernel"] = "bf16 8192^3 GEMM (hipBLASLt via torch.matmul)"
        if "measured_peak" in r:
            r["frac_of_measured"] = round(achieved / r["measured_peak"], 4)
    kernel = "k_attend_prefill" if phase == "encode" and w.dtype == "bf16" else "k_attend_rows"
    call = "infllm_attend"
    if phase == "decode" and fused:
        kernel, call = "k_select_attend", "infllm_select_attend"
    r["traffic"] = stored_traffic(kernel, w.name)
    r["kernel"] = "%s (%s)" % (call, kernel)
    r["avg_launch_us"] = round(attn_ms * 1e3, 2)
    # the same work over the kernel's average duration in the committed
    # rocprofv3 trace (another run, on another box): what the profile gives
    prof_us = stored_profile_us(kernel, w.name)
    r["profile_avg_launch_us"] = prof_us
    r["frac_from_profile"] = (round(r["frac"] * attn_ms * 1e3 / prof_us, 4)
                              if prof_us else None)
    r["launches_per_step"] = n_calls
    r["launch_timing"] = ("HIP events on the launch stream around each timed step's "
                          "attention launches (back to back), divided by their count; "
                          "dispatch gaps between launches included")
    return r


# Every workload of the scope, in the order the default run measures them;
# the first is the headline (the chunked encoding of a Llama-3-8B layer).
ALL_WORKLOADS = ["llama3_8b_32k_encode", "llama3_8b_128k_decode", "llama3_8b_1m_decode",
                 "mistral_7b_64k_tokens", "mistral_7b_64k_mean", "tiny_f32"]


def offload_decode(pipe: Pipeline, slots: int, steps: int) -> dict:
    """The decode pass with the context's K/V in pinned host memory (the
    GPU holding only the initial tokens, a ring of the window and a cache of
    `slots` units per (sequence, KV head)): per step the selection, the
    fetch (misses copied in by the GPU over the host link) and the
    attention over the cache; layer 0, a fresh (empty) cache, the first
    `steps` decode positions.  The last step's output is checked bit for
    bit against the resident attention."""
    w, cfg, inp = pipe.w, pipe.cfg, pipe.inp
    k, v = pipe.layers[0]["k"], pipe.layers[0]["v"]
    b, Hkv, d, B = w.batch, w.n_kv_heads, w.head_dim, w.block
    t = time.time()
    k_host = torch.empty(k.shape, dtype=k.dtype, pin_memory=True)
    v_host = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
    k_host.copy_(k)
    v_host.copy_(v)
    pin_s = time.time() - t
    n_init, W = w.n_init, w.window
    t_last = w.n_ctx + steps - 1
    local_cap = n_init + W + steps + 64
    R = local_cap - n_init
    kl = torch.zeros((b, Hkv, local_cap, d), dtype=k.dtype, device="cuda")
    vl = torch.zeros_like(kl)
    kl[:, :, :n_init] = k[:, :, :n_init]
    vl[:, :, :n_init] = v[:, :, :n_init]
    pp = torch.arange(max(n_init, t_last - R + 1), t_last + 1, device="cuda")
    rows = n_init + (pp - n_init) % R
    kl[:, :, rows] = k[:, :, pp]
    vl[:, :, rows] = v[:, :, pp]
    cache_k = torch.empty((b, Hkv, slots, B, d), dtype=k.dtype, device="cuda")
    cache_v = torch.empty_like(cache_k)
    ws = F.workspace(cfg, F.INFLLM_CALL_ATTEND, b, 0, 1, 1)
    out = torch.empty_like(inp["q_dec"])
    sel = pipe.sel_dec

    def run(state, n, fetch_only=False):
        for s in range(n):
            F.infllm_cache_fetch(cfg, sel[s], pipe.U, s + 1, k_host, v_host, cache_k, cache_v,
                                 state)
            if not fetch_only:
                F.infllm_attend_cached(cfg, inp["q_dec"], s, w.n_ctx + s, 1, kl, vl, k.shape[2],
                                       sel[s], pipe.U, cache_k, cache_v, state, out, None, s,
                                       ws=ws)

    for s in range(steps):
        pipe._select(inp["q_dec"], s, w.n_ctx + s, 1, sel[s], pipe.dec_score_ws, 0)
    run(F.cache_state(cfg, b, pipe.U, slots), 2)            # warm-up
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    state = F.cache_state(cfg, b, pipe.U, slots)
    e[0].record()
    for s in range(steps):
        pipe._select(inp["q_dec"], s, w.n_ctx + s, 1, sel[s], pipe.dec_score_ws, 0)
    run(state, steps)
    e[1].record()
    torch.cuda.synchronize()
    hits, misses = F.infllm_cache_stats(state)
    e[2].record()
    run(F.cache_state(cfg, b, pipe.U, slots), steps, fetch_only=True)
    e[3].record()
    torch.cuda.synchronize()
    o_res = torch.empty_like(out)
    F.infllm_attend(cfg, inp["q_dec"], steps - 1, w.n_ctx + steps - 1, 1, 1, k, v,
                    sel[steps - 1], o_res, None, steps - 1, pipe.dec_attn_ws)
    torch.cuda.synchronize()
    same = bool(torch.equal(out[:, :, steps - 1], o_res[:, :, steps - 1]))
    ms = e[0].elapsed_time(e[1]) / steps
    fetch_ms = e[2].elapsed_time(e[3]) / steps
    unit_bytes = 2 * B * d * k.element_size()           # K and V of one unit
    host_bytes = misses * unit_bytes / steps
    return {"form": "K/V in pinned host memory; per step select, fetch (GPU loads over the "
                    "host link) and attention over the unit cache; fresh cache, layer 0",
            "slots": slots, "steps": steps, "ms_per_decode_step": round(ms, 4),
            "hit_ratio": round(hits / max(1, hits + misses), 4),
            "misses_per_step": round(misses / steps, 2),
            "host_bytes_per_step": int(host_bytes),
            "fetch_ms_per_step": round(fetch_ms, 4),
            "host_link_GB_s": round(host_bytes / (fetch_ms * 1e-3) / 1e9, 2),
            "gpu_resident_bytes": int((kl.numel() + vl.numel() + cache_k.numel() * 2)
                                      * k.element_size()),
            "pin_seconds": round(pin_s, 2),
            "last_step_equals_resident": same}


def measure(w: synth.Workload, args, peaks, cpu_seconds: float) -> dict:
    """One workload: settle, warm up, time args.steps steps; the record (the
    bench line's fields for this workload)."""
    decode_only = w.chunk == 0
    layers = (args.layers or 4) if decode_only else 1
    pipe = (StreamPipeline(w, layers=layers, rope_theta=args.rope_theta) if args.stream else
            Pipeline(w, layers=layers, fused_step=not args.separate_decode,
                     rope_theta=args.rope_theta))
    if not pipe.encode:
        pipe.build_all()        # decode-only: the pools are built once, beforehand
    # Untimed settling before the warm-up steps: the GPU's clocks ramp up
    # over the first ~100 ms of sustained work (a 2-step warm-up left the
    # 32K encoding step ~6% slower than steady state), so steps run until
    # args.settle seconds have passed.
    settle_steps = 0
    t_settle = time.time()
    while time.time() - t_settle < args.settle:
        pipe.step()
        torch.cuda.synchronize()
        settle_steps += 1
    for _ in range(args.warmup):
        pipe.step()
    torch.cuda.synchronize()

    # The timed steps carry events only at their phase boundaries; each
    # event costs the stream a few microseconds, a few per step.
    marks = {}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        pipe.step(marks)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    def span_ms(a, b):
        return float(np.mean([x.elapsed_time(y) for x, y in zip(marks[a], marks[b])]))

    work = pipe.work()
    tokens = sum(v[0] for v in work.values())
    phase = "encode" if pipe.encode else "decode"
    rec = {
        "metric": "attended KV tokens/s (InfLLM attention step, Llama-3-8B layer)",
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "attended KV tokens/s",
        "steps": args.steps, "warmup": args.warmup,
        "settle": {"seconds": args.settle, "steps": settle_steps},
        "ms_per_step": round(ms_step, 4),
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "config": {"workload": w.name, "batch": w.batch, "n_ctx": w.n_ctx,
                   "heads": "%dq/%dkv" % (w.n_q_heads, w.n_kv_heads), "head_dim": w.head_dim,
                   "chunk": w.chunk, "decode_steps": w.decode_steps, "block": w.block,
                   "n_init": w.n_init, "window": w.window, "rep_k": w.rep_k, "top_k": w.top_k,
                   "rep_mode": w.rep_mode, "layers": layers,
                   "attended_tokens_per_step": tokens},
        "roofline": (roofline(w, "encode", work["encode"], span_ms("enc_sel", "enc_end"), 1,
                              peaks)
                     if phase == "encode" else
                     roofline(w, "decode", work["decode"],
                              span_ms("dec_sel", "dec_end") / w.decode_steps, w.decode_steps,
                              peaks, getattr(pipe, "fused", False))),
    }
    if args.rope_theta > 0:
        # the committed profiles cover the as-given kernels, not the turning ones
        rec["config"]["rope_theta"] = args.rope_theta
        rec["roofline"].update(traffic=None, profile_avg_launch_us=None, frac_from_profile=None)
    if args.stream:
        rec["config"]["stream"] = {"lengths": pipe.lens, "pool_units": pipe.U,
                                   "unit_build_calls_per_step": pipe.n_builds * len(pipe.layers)}
        rec["roofline"]["traffic"] = None      # counters were taken on the fixed-pool form
    if pipe.decode:
        # one decode step = score + top-k + attention for one token position;
        # the decode pass of a step: from the end of its encoding pass
        ms_decode = span_ms("enc_end", "dec_end") if pipe.encode else ms_step
        rec["ms_per_decode_step"] = round(ms_decode / w.decode_steps, 5)
        rec["decode_tokens_per_s"] = round(work["decode"][0] / (ms_decode * 1e-3), 1)
        rec["decode_form"] = ("one launch per step (infllm_select_attend)"
                              if getattr(pipe, "fused", False) else
                              "selection and attention launches per step")
        # the whole step against HBM: every byte the step must move (K/V rows
        # attended, queries and outputs, every unit row scored) over the
        # step's own time
        step_bytes = work["decode"][2] / w.decode_steps
        if not getattr(pipe, "fused", False):
            step_bytes += w.batch * w.n_kv_heads * pipe.U * (w.head_dim + 1) * 4
        gbs = step_bytes / (ms_decode / w.decode_steps * 1e-3) / 1e9
        rec["decode_step_hbm"] = {"bytes": int(step_bytes), "GB_s": round(gbs, 1),
                                  "frac": round(gbs / PEAK_HBM_GBS, 4), "peak": PEAK_HBM_GBS}
        if pipe.encode:
            rec["decode_roofline"] = roofline(w, "decode", work["decode"],
                                              span_ms("dec_sel", "dec_end") / w.decode_steps,
                                              w.decode_steps, peaks, pipe.fused)
            if args.rope_theta > 0:
                rec["decode_roofline"].update(traffic=None, profile_avg_launch_us=None,
                                              frac_from_profile=None)
    if (pipe.decode and not pipe.encode and not args.stream and args.offload_slots > 0
            and w.n_ctx >= (1 << 20)):
        rec["offload"] = offload_decode(pipe, args.offload_slots,
                                        min(args.offload_steps, w.decode_steps))
    if pipe.encode and not args.stream and not args.no_sequential:
        # the same encoding pass chunk by chunk (one call of each kind per
        # chunk), as the pages process a context
        n_seq = max(1, min(args.steps, 5))
        pipe.step_sequential()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_seq):
            pipe.step_sequential()
        e1.record()
        torch.cuda.synchronize()
        ms_seq = e0.elapsed_time(e1) / n_seq
        enc_ms = ms_step - (span_ms("enc_end", "dec_end") if pipe.decode else 0.0)
        rec["sequential_encode"] = {
            "form": "build, then score + top-k + attention per chunk, %d chunks one after another"
                    % pipe.n_chunks,
            "ms_per_pass": round(ms_seq, 4), "batched_ms_per_pass": round(enc_ms, 4),
            "tokens_per_s": round(work["encode"][0] / (ms_seq * 1e-3), 1)}
    if args.calibration_copy > 0:
        n = args.calibration_copy << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                       # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        rec["calibration_copy_bytes"] = n
    if cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(w, pipe, cpu_seconds)
    del pipe
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None, choices=sorted(synth.WORKLOADS),
                    help="measure this workload only (default: the 32K encoding headline, then "
                         "every other workload as a sub-record of the same line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-decode", action="store_true",
                    help="decode with infllm_select_units + infllm_attend (two launches per "
                         "step) instead of infllm_select_attend")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring what plain library kernels reach (read, GEMM)")
    ap.add_argument("--layers", type=int, default=None,
                    help="decode workloads: rotate the decode steps over this many layers' "
                         "K/V and unit pools (default 4, so that a step's K/V is not still in "
                         "the 256 MB last-level cache from the step before; 1 for the "
                         "single-layer figure); encoding workloads use one layer")
    ap.add_argument("--settle", type=float, default=1.0, metavar="SECONDS",
                    help="untimed steps for this long before the warm-up steps, so that the "
                         "GPU clocks reach steady state (0 to skip)")
    ap.add_argument("--stream", action="store_true",
                    help="decode workloads: serving form -- ragged sequence lengths, a device "
                         "position per sequence, units added to the pools as they leave the "
                         "window (streaming unit build)")
    ap.add_argument("--no-sequential", action="store_true",
                    help="encoding workloads: skip the chunk-by-chunk pass (profiling runs, "
                         "so that every attention launch in the trace is the one-call pass)")
    ap.add_argument("--offload-slots", type=int, default=64,
                    help="1M-token decode: also run the decode pass with the K/V in pinned host "
                         "memory and a GPU cache of this many units per (sequence, KV head) "
                         "(0 to skip)")
    ap.add_argument("--offload-steps", type=int, default=16,
                    help="decode steps of that pass (each miss moves a unit over the host link)")
    ap.add_argument("--rope-theta", type=float, default=0.0, metavar="THETA",
                    help="RoPE base: the attention re-positions q and k inside each working "
                         "context (timing only: no oracle baseline, no offload record)")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run one plain device copy of MIB MiB (untimed), the "
                         "reference kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path runs on a single MI355X with the whole unit "
              "pool resident; runs on %d GPUs are not part of this benchmark" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.rope_theta < 0:
        print("--rope-theta must be >= 0", file=sys.stderr)
        sys.exit(2)
    if args.rope_theta > 0:
        # the oracle baseline and the offload record time the as-given form
        args.no_cpu_baseline, args.offload_slots = True, 0
    torch.cuda.set_device(0)
    names = [args.workload] if args.workload else ALL_WORKLOADS
    if args.stream and any(synth.WORKLOADS[n].chunk > 0 for n in names):
        print("--stream applies to decode workloads (name one with --workload)", file=sys.stderr)
        sys.exit(2)
    peaks = None if args.no_peaks else measure_peaks()
    cpu = 0.0 if args.no_cpu_baseline else CPU_SAMPLE_SECONDS
    head = measure(synth.WORKLOADS[names[0]], args, peaks, cpu)
    line = {"metric": head.pop("metric"), "value": head.pop("value"), "unit": head.pop("unit"),
            "n_gpus": 1}
    line.update({k: head[k] for k in ("steps", "warmup", "settle", "ms_per_step")})
    line.update({"higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                 "dtype": head["dtype"], "data": "synthetic"})
    for k, v in head.items():
        if k not in line:
            line[k] = v
    if len(names) > 1:
        # the other workloads of the scope, each measured the same way (a
        # shorter oracle sample each)
        line["workloads"] = {}
        for n in names[1:]:
            print("measuring %s" % n, file=sys.stderr, flush=True)
            line["workloads"][n] = measure(synth.WORKLOADS[n], args, peaks, cpu / 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
