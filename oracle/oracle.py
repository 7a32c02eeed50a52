"""Oracle wrapper -- TEST INFRASTRUCTURE ONLY.

Python access to ``infllm_oracle.c``, the plain fp64 CPU statement of
InfLLM's context-memory attention step.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
module.  It imports nothing from the HIP product package and the product
package never imports it.

Per-(sequence, KV head) functions take CPU tensors:
  qg   [G, n, d]  the G query heads of one KV head (fp32 or bf16),
  k, v [n, d]     keys/values, row p = absolute position p,
and return fp64 numpy arrays (int32 for indices).  The ``*_all`` drivers
loop those over batch and KV heads for [b, H, n, d] tensors.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "infllm_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

_i32, _i64, _f64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p


def build() -> str:
    """Compile the oracle with gcc (plain C, OpenMP); returns the .so path."""
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, _SO)
    return _SO


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        so = os.environ.get("INFLLM_ORACLE_SO")     # a mutant, for the pin meta-test
        if so is None:
            so = _SO
            if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(so)
        L.orc_num_threads.restype = _i32
        L.orc_num_units.restype = _i64
        L.orc_num_units.argtypes = [_i64, _i32, _i32]
        L.orc_unit_keys.argtypes = [_i64, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        L.orc_num_eligible.restype = _i64
        L.orc_num_eligible.argtypes = [_i64, _i64, _i32, _i32, _i32]
        L.orc_rep_score.restype = _f64
        L.orc_rep_score.argtypes = [_vp, _i64, _i32, _vp, _i32, _i32, _i64, _i32, _i64]
        L.orc_build_tokens.argtypes = [_vp, _i64, _i32, _vp, _i32, _i32, _i64, _i32, _i32,
                                       _i32, _i32, _i64, _i64, _vp, _vp, _vp]
        L.orc_build_mean.argtypes = [_vp, _i32, _i32, _i32, _i32, _i64, _i64, _vp]
        L.orc_score_units.argtypes = [_vp, _i64, _i32, _i32, _i32, _i64, _vp, _i64, _i64, _vp]
        L.orc_topk.argtypes = [_vp, _i64, _i64, _i32, _vp]
        L.orc_in_working_context.restype = ctypes.c_int
        L.orc_in_working_context.argtypes = [_i64, _i64, _vp, _i32, _i32, _i32, _i32]
        L.orc_working_context.restype = _i64
        L.orc_working_context.argtypes = [_i64, _vp, _i32, _i32, _i32, _i32, _vp]
        L.orc_attend.argtypes = [_vp, _i64, _i32, _i64, _i64, _vp, _vp, _i32, _i32, _vp,
                                 _i32, _i32, _i32, _i32, _f64, _vp, _vp]
        L.orc_context_pos.restype = _i64
        L.orc_context_pos.argtypes = [_i64, _i64, _vp, _i32, _i32, _i32, _i32]
        _LIB = L
    return _LIB


def num_threads() -> int:
    return int(lib().orc_num_threads())


# --------------------------------------------------------------------------
# marshalling
def _host(t: torch.Tensor) -> torch.Tensor:
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("oracle inputs are fp32 or bf16, got %s" % t.dtype)
    return t.contiguous()


def _dt(t: torch.Tensor) -> int:
    return 0 if t.dtype == torch.float32 else 1


def _p(a) -> ctypes.c_void_p:
    if isinstance(a, torch.Tensor):
        return ctypes.c_void_p(a.data_ptr())
    return ctypes.c_void_p(a.ctypes.data)


def _i32arr(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# --------------------------------------------------------------------------
# unit table
def num_units(n_ctx: int, B: int, n_init: int) -> int:
    return int(lib().orc_num_units(n_ctx, B, n_init))


def unit_keys(u: int, B: int, n_init: int) -> tuple[int, int]:
    lo, hi = _i64(), _i64()
    lib().orc_unit_keys(u, B, n_init, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def num_eligible(t_last: int, U: int, B: int, n_init: int, W: int) -> int:
    return int(lib().orc_num_eligible(t_last, U, B, n_init, W))


# --------------------------------------------------------------------------
# per (sequence, KV head)
def rep_score(qg, k, n_ctx: int, W: int, p: int) -> float:
    qg, k = _host(qg), _host(k)
    G, n, d = qg.shape
    return float(lib().orc_rep_score(_p(qg), n * d, G, _p(k), d, _dt(k), n_ctx, W, p))


def build_tokens(qg, k, n_ctx: int, B: int, n_init: int, W: int, r_k: int,
                 u_lo: int = 0, u_hi: int | None = None):
    """-> rep_idx int32 [n, r_k], repr f64 [n, d], key_scores f64 [n, B]."""
    qg, k = _host(qg), _host(k)
    G, nq, d = qg.shape
    if u_hi is None:
        u_hi = num_units(n_ctx, B, n_init)
    n = u_hi - u_lo
    rep_idx = np.zeros((n, r_k), np.int32)
    repr_ = np.zeros((n, d), np.float64)
    ks = np.zeros((n, B), np.float64)
    if n > 0:
        lib().orc_build_tokens(_p(qg), nq * d, G, _p(k), d, _dt(k), n_ctx, B, n_init, W, r_k,
                               u_lo, u_hi, _p(rep_idx), _p(repr_), _p(ks))
    return rep_idx, repr_, ks


def build_mean(k, B: int, n_init: int, u_lo: int, u_hi: int) -> np.ndarray:
    k = _host(k)
    d = k.shape[1]
    repr_ = np.zeros((u_hi - u_lo, d), np.float64)
    if u_hi > u_lo:
        lib().orc_build_mean(_p(k), d, _dt(k), B, n_init, u_lo, u_hi, _p(repr_))
    return repr_


def score_units(qg_chunk, repr_, e: int) -> np.ndarray:
    qg = _host(qg_chunk)
    G, L, d = qg.shape
    r = np.ascontiguousarray(np.asarray(repr_, np.float64))
    U = r.shape[0]
    out = np.zeros(U, np.float64)
    lib().orc_score_units(_p(qg), L * d, G, d, _dt(qg), L, _p(r), U, e, _p(out))
    return out


def topk(scores, e: int, k_m: int) -> np.ndarray:
    s = np.ascontiguousarray(np.asarray(scores, np.float64))
    sel = np.zeros(max(k_m, 0), np.int32)
    if k_m > 0:
        lib().orc_topk(_p(s), s.shape[0], e, k_m, _p(sel))
    return sel


def in_working_context(p: int, t: int, sel, B: int, n_init: int, W: int) -> bool:
    s = _i32arr(sel)
    return bool(lib().orc_in_working_context(p, t, _p(s), s.shape[0], B, n_init, W))


def working_context(t: int, sel, B: int, n_init: int, W: int) -> np.ndarray:
    s = _i32arr(sel)
    n = int(lib().orc_working_context(t, _p(s), s.shape[0], B, n_init, W, None))
    out = np.zeros(max(n, 1), np.int64)
    lib().orc_working_context(t, _p(s), s.shape[0], B, n_init, W, _p(out))
    return out[:n]


def attend(qg, t0: int, k, v, sel, B: int, n_init: int, W: int, rope_theta: float = 0.0):
    """Queries rows 0..L-1 of qg sit at positions t0..t0+L-1.  rope_theta > 0:
    q and k are rotated at their absolute positions and the attention re-
    indexes them to working-context positions.
    -> out f64 [G, L, d], lse f64 [G, L]."""
    qg, k, v = _host(qg), _host(k), _host(v)
    G, L, d = qg.shape
    s = _i32arr(sel)
    out = np.zeros((G, L, d), np.float64)
    lse = np.zeros((G, L), np.float64)
    if L > 0:
        lib().orc_attend(_p(qg), L * d, G, t0, L, _p(k), _p(v), d, _dt(k), _p(s), s.shape[0],
                         B, n_init, W, float(rope_theta), _p(out), _p(lse))
    return out, lse


def context_pos(p: int, t0: int, sel, B: int, n_init: int, W: int) -> int:
    """Working-context position of token p for the chunk starting at t0."""
    s = _i32arr(sel)
    return int(lib().orc_context_pos(p, t0, _p(s), s.shape[0], B, n_init, W))


# --------------------------------------------------------------------------
# drivers over [b, H, n, d] tensors
def build_units_all(q, k, n_ctx: int, *, B: int, n_init: int, W: int, r_k: int,
                    mode: str = "tokens"):
    """q [b,H_q,>=n_ctx,d], k [b,H_kv,>=n_ctx,d] ->
    rep_idx [b,H_kv,U,r_k] (None for mean), repr [b,H_kv,U,d], key_scores (None for mean)."""
    b, Hq, _, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    U = num_units(n_ctx, B, n_init)
    repr_ = np.zeros((b, Hkv, U, d))
    if mode == "mean":
        for bi in range(b):
            for h in range(Hkv):
                repr_[bi, h] = build_mean(k[bi, h, :n_ctx], B, n_init, 0, U)
        return None, repr_, None
    rep_idx = np.zeros((b, Hkv, U, r_k), np.int32)
    ks = np.zeros((b, Hkv, U, B))
    for bi in range(b):
        for h in range(Hkv):
            ri, rr, kk = build_tokens(q[bi, h * G:(h + 1) * G, :n_ctx], k[bi, h, :n_ctx],
                                      n_ctx, B, n_init, W, r_k)
            rep_idx[bi, h], repr_[bi, h], ks[bi, h] = ri, rr, kk
    return rep_idx, repr_, ks


def select_all(q_chunk, t0: int, repr_, *, B: int, n_init: int, W: int, k_m: int):
    """One chunk (q_chunk [b,H_q,L,d] at positions t0..) ->
    scores f64 [b,H_kv,U], sel int32 [b,H_kv,k_m], e."""
    b, Hq, L, d = q_chunk.shape
    Hkv, U = repr_.shape[1], repr_.shape[2]
    G = Hq // Hkv
    e = num_eligible(t0 + L - 1, U, B, n_init, W)
    scores = np.zeros((b, Hkv, U))
    sel = np.zeros((b, Hkv, k_m), np.int32)
    for bi in range(b):
        for h in range(Hkv):
            scores[bi, h] = score_units(q_chunk[bi, h * G:(h + 1) * G], repr_[bi, h], e)
            sel[bi, h] = topk(scores[bi, h], e, k_m)
    return scores, sel, e


def attend_all(q_chunk, t0: int, k, v, sel, *, B: int, n_init: int, W: int,
               rope_theta: float = 0.0):
    """q_chunk [b,H_q,L,d] at positions t0.., k/v [b,H_kv,n,d], sel [b,H_kv,k_m]
    -> out f64 [b,H_q,L,d], lse f64 [b,H_q,L]."""
    b, Hq, L, d = q_chunk.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((b, Hq, L, d))
    lse = np.zeros((b, Hq, L))
    for bi in range(b):
        for h in range(Hkv):
            o, l = attend(q_chunk[bi, h * G:(h + 1) * G], t0, k[bi, h], v[bi, h], sel[bi, h],
                          B, n_init, W, rope_theta)
            out[bi, h * G:(h + 1) * G], lse[bi, h * G:(h + 1) * G] = o, l
    return out, lse
