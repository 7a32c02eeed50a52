"""ctypes binding of libinfllm.so (include/infllm.h), same call names.

Argument marshalling only: shapes and dtypes of torch tensors are checked,
then data pointers, sizes and the current HIP stream are handed to the C
ABI, which does every step of the work in HIP kernels.  There is no
fallback: if the library is missing or a call fails, an exception says so.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinfllm.so")

INFLLM_OK, INFLLM_ERR_INVALID_ARG, INFLLM_ERR_UNSUPPORTED, INFLLM_ERR_WORKSPACE, INFLLM_ERR_HIP = \
    0, -1, -2, -3, -4
INFLLM_F32, INFLLM_BF16 = 0, 1
INFLLM_REP_TOKENS, INFLLM_REP_MEAN = 0, 1
INFLLM_CALL_BUILD, INFLLM_CALL_SCORE, INFLLM_CALL_TOPK, INFLLM_CALL_ATTEND = 0, 1, 2, 3
INFLLM_CALL_BUILD_RANGE, INFLLM_CALL_SELECT, INFLLM_CALL_BUILD_QSUM = 4, 5, 6
INFLLM_CALL_SELECT_ATTEND = 7

EXPORTED = ("infllm_num_units", "infllm_num_eligible", "infllm_workspace_size",
            "infllm_build_units", "infllm_build_units_range", "infllm_build_units_qsum",
            "infllm_score_units", "infllm_score_units_qsum",
            "infllm_score_units_varlen", "infllm_select_units", "infllm_topk_units",
            "infllm_attend", "infllm_attend_varlen", "infllm_select_attend",
            "infllm_select_attend_static",
            "infllm_workspace_layout", "infllm_workspace_status", "infllm_step_plan",
            "infllm_cache_state_size", "infllm_cache_fetch", "infllm_attend_cached",
            "infllm_cache_stats", "infllm_status_string", "infllm_abi_version")


ABI_VERSION = 2   # INFLLM_ABI_VERSION of include/infllm.h


class infllm_config(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("n_init", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rep_k", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("rep_mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_double)]


class InfllmError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (call, status_string(status), status))


_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_cfgp = ctypes.POINTER(infllm_config)
_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libinfllm.so is not built (run: python -m block_level_kv_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.infllm_num_units.restype = _i32
        L.infllm_num_units.argtypes = [_cfgp, _i64]
        L.infllm_num_eligible.restype = _i32
        L.infllm_num_eligible.argtypes = [_cfgp, _i64, _i32]
        L.infllm_workspace_size.restype = _sz
        L.infllm_workspace_size.argtypes = [_cfgp, _i32, _i32, _i64, _i32, _i32]
        L.infllm_build_units.restype = _i32
        L.infllm_build_units.argtypes = [_cfgp, _i32, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp,
                                         _sz, _vp]
        L.infllm_build_units_qsum.restype = _i32
        L.infllm_build_units_qsum.argtypes = [_cfgp, _i32, _vp, _i64, _vp, _i64, _i64, _vp, _vp,
                                              _vp, _vp, _sz, _vp]
        L.infllm_score_units_qsum.restype = _i32
        L.infllm_score_units_qsum.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _i32, _i32, _vp, _i32,
                                              _vp, _vp]
        L.infllm_build_units_range.restype = _i32
        L.infllm_build_units_range.argtypes = [_cfgp, _i32, _vp, _i64, _vp, _i64, _i64, _i32, _i32,
                                               _i32, _vp, _vp, _vp, _sz, _vp]
        L.infllm_score_units.restype = _i32
        L.infllm_score_units.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _i32,
                                         _vp, _vp, _sz, _vp]
        L.infllm_score_units_varlen.restype = _i32
        L.infllm_score_units_varlen.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _vp, _i32, _i32, _vp,
                                                _i32, _vp, _vp, _sz, _vp]
        L.infllm_attend_varlen.restype = _i32
        L.infllm_attend_varlen.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _vp, _i32, _i32, _vp, _vp,
                                           _i64, _vp, _vp, _vp, _i64, _i64, _vp, _sz, _vp]
        L.infllm_cache_state_size.restype = _sz
        L.infllm_cache_state_size.argtypes = [_cfgp, _i32, _i32, _i32]
        L.infllm_cache_fetch.restype = _i32
        L.infllm_cache_fetch.argtypes = [_cfgp, _i32, _i32, _vp, _i32, _i64, _vp, _vp, _i64, _vp,
                                         _vp, _i32, _vp, _vp]
        L.infllm_attend_cached.restype = _i32
        L.infllm_attend_cached.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                                           _i64, _i64, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp,
                                           _i64, _i64, _vp, _sz, _vp]
        L.infllm_cache_stats.restype = _i32
        L.infllm_cache_stats.argtypes = [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64), _vp]
        L.infllm_select_units.restype = _i32
        L.infllm_select_units.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _i64, _vp, _i32, _i32, _vp,
                                          _i32, _vp, _vp, _vp, _sz, _vp]
        L.infllm_select_attend.restype = _i32
        L.infllm_select_attend.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _i32,
                                           _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _vp,
                                           _sz, _vp]
        L.infllm_select_attend_static.restype = _i32
        L.infllm_select_attend_static.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _i64, _vp, _i32, _vp,
                                                  _i32, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i64,
                                                  _i64, _vp]
        L.infllm_topk_units.restype = _i32
        L.infllm_topk_units.argtypes = [_cfgp, _i32, _i32, _vp, _i32, _vp, _vp, _sz, _vp]
        L.infllm_attend.restype = _i32
        L.infllm_attend.argtypes = [_cfgp, _i32, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _i64,
                                    _vp, _vp, _vp, _i64, _i64, _vp, _sz, _vp]
        L.infllm_workspace_layout.restype = _i32
        L.infllm_workspace_layout.argtypes = [_cfgp, _i32, _i32, _i64, _i32, _i32,
                                              ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                              ctypes.POINTER(_sz)]
        L.infllm_step_plan.restype = _i32
        L.infllm_step_plan.argtypes = [_cfgp, _i32, _i32, _i32, ctypes.POINTER(_i32)]
        L.infllm_workspace_status.restype = _i32
        L.infllm_workspace_status.argtypes = [_vp, _sz, ctypes.POINTER(_i32), _vp]
        L.infllm_status_string.restype = ctypes.c_char_p
        L.infllm_status_string.argtypes = [_i32]
        L.infllm_abi_version.restype = _i32
        if L.infllm_abi_version() != ABI_VERSION:   # infllm_config layout changed
            raise RuntimeError("libinfllm.so has ABI version %d, this binding needs %d "
                               "(rebuild: python -m block_level_kv_amd.build)"
                               % (L.infllm_abi_version(), ABI_VERSION))
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().infllm_status_string(status).decode()


def make_config(*, n_q_heads: int, n_kv_heads: int, head_dim: int, block: int, n_init: int,
                window: int, rep_k: int, top_k: int, rep_mode: int = INFLLM_REP_TOKENS,
                dtype: int = INFLLM_BF16, rope_theta: float = 0.0) -> infllm_config:
    return infllm_config(n_q_heads, n_kv_heads, head_dim, block, n_init, window, rep_k, top_k,
                         rep_mode, dtype, rope_theta)


# ------------------------------------------------------------------ helpers
def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


# the raw current-stream handle of a device, without building a Stream
# object (a few microseconds per call otherwise)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, t: torch.Tensor) -> int | None:
    """The stream to launch on: `stream` if given, else the current stream of
    tensor t's device."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.get_device())
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype_of(cfg: infllm_config) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == INFLLM_BF16 else torch.float32


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype != dtype or t.dim() != ndim or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %dD %s CUDA/HIP tensor, got %s %s %s" %
                         (name, ndim, dtype, t.dtype, tuple(t.shape), t.device))


def _ws(t: torch.Tensor | None) -> tuple[int | None, int]:
    if t is None:
        return None, 0
    return t.data_ptr(), t.numel() * t.element_size()


def _raise(call: str, status: int) -> None:
    if status != INFLLM_OK:
        raise InfllmError(call, status)


# ------------------------------------------------------------------ calls
def infllm_num_units(cfg: infllm_config, n_ctx: int) -> int:
    return int(lib().infllm_num_units(ctypes.byref(cfg), n_ctx))


def infllm_num_eligible(cfg: infllm_config, t_last: int, n_units: int) -> int:
    return int(lib().infllm_num_eligible(ctypes.byref(cfg), t_last, n_units))


def infllm_workspace_size(cfg: infllm_config, call: int, batch: int, n: int = 0,
                          chunk_len: int = 0, n_chunks: int = 0) -> int:
    return int(lib().infllm_workspace_size(ctypes.byref(cfg), call, batch, n, chunk_len, n_chunks))


def infllm_workspace_layout(cfg: infllm_config, call: int, batch: int, n: int = 0,
                            chunk_len: int = 0, n_chunks: int = 0) -> tuple[int, int, int]:
    """(counters_begin, counters_end, total) bytes of a call's workspace."""
    b, e, t = _sz(0), _sz(0), _sz(0)
    _raise("infllm_workspace_layout", lib().infllm_workspace_layout(
        ctypes.byref(cfg), call, batch, n, chunk_len, n_chunks, ctypes.byref(b), ctypes.byref(e),
        ctypes.byref(t)))
    return b.value, e.value, t.value


def infllm_step_plan(cfg: infllm_config, batch: int, n_units: int, n_pos: int = 1) -> dict:
    """How infllm_select_attend runs a step: one launch or the two calls, and
    the one launch's shape."""
    p = (_i32 * 7)()
    _raise("infllm_step_plan", lib().infllm_step_plan(ctypes.byref(cfg), batch, n_units, n_pos, p))
    keys = ("fused", "n_splits", "s_score", "units_per", "cand", "w_score", "w_unit")
    return {k: int(v) for k, v in zip(keys, p)}


def infllm_workspace_status(ws: torch.Tensor, stream=None) -> int:
    """Waits of the one-launch decode step that hit their bound (synchronises)."""
    n = _i32(0)
    _raise("infllm_workspace_status", lib().infllm_workspace_status(
        ws.data_ptr(), ws.numel() * ws.element_size(), ctypes.byref(n), _stream(stream, ws)))
    return n.value


def workspace(cfg: infllm_config, call: int, batch: int, n: int = 0, chunk_len: int = 0,
              n_chunks: int = 0, device="cuda") -> torch.Tensor | None:
    """A caller-owned, zero-filled workspace tensor of the size `call` needs
    (None if 0).  Zero-filled because the score and attention workspaces
    carry arrival counters that must start at zero (and stay zero between
    calls)."""
    size = infllm_workspace_size(cfg, call, batch, n, chunk_len, n_chunks)
    if size == 0:
        return None
    return torch.zeros(size, dtype=torch.uint8, device=device)


def infllm_build_units(cfg, q, k, n_ctx: int, rep_idx, unit_repr, ws=None, stream=None) -> None:
    dt = _dtype_of(cfg)
    if cfg.rep_mode == INFLLM_REP_TOKENS:
        _check(q, "q", dt, 4)
        _check(rep_idx, "rep_idx", torch.int32, 4)
    _check(k, "k", dt, 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    batch = k.shape[0]
    U = infllm_num_units(cfg, n_ctx)
    if tuple(unit_repr.shape) != (batch, cfg.n_kv_heads, U, cfg.head_dim):
        raise ValueError("unit_repr must be [batch, H_kv, U=%d, d]" % U)
    if rep_idx is not None and tuple(rep_idx.shape) != (batch, cfg.n_kv_heads, U, cfg.rep_k):
        raise ValueError("rep_idx must be [batch, H_kv, U=%d, r_k]" % U)
    q_cap = q.shape[2] if q is not None else 0
    wp, wb = _ws(ws)
    _raise("infllm_build_units", lib().infllm_build_units(
        ctypes.byref(cfg), batch, _ptr(q), q_cap, k.data_ptr(), k.shape[2], n_ctx,
        _ptr(rep_idx), unit_repr.data_ptr(), wp, wb, _stream(stream, k)))


def infllm_build_units_qsum(cfg, q, k, n_ctx: int, rep_idx, unit_repr, block_qsum, ws=None,
                            stream=None) -> None:
    """infllm_build_units that also writes the fp64 block query sums
    [batch, H_kv, ceil(n_ctx/B), d]."""
    dt = _dtype_of(cfg)
    _check(q, "q", dt, 4)
    _check(k, "k", dt, 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    _check(block_qsum, "block_qsum", torch.float64, 4)
    if cfg.rep_mode == INFLLM_REP_TOKENS:
        _check(rep_idx, "rep_idx", torch.int32, 4)
    batch = k.shape[0]
    U = infllm_num_units(cfg, n_ctx)
    nb = (n_ctx + cfg.block - 1) // cfg.block
    if tuple(unit_repr.shape) != (batch, cfg.n_kv_heads, U, cfg.head_dim):
        raise ValueError("unit_repr must be [batch, H_kv, U=%d, d]" % U)
    if tuple(block_qsum.shape) != (batch, cfg.n_kv_heads, nb, cfg.head_dim):
        raise ValueError("block_qsum must be [batch, H_kv, %d, d]" % nb)
    wp, wb = _ws(ws)
    _raise("infllm_build_units_qsum", lib().infllm_build_units_qsum(
        ctypes.byref(cfg), batch, q.data_ptr(), q.shape[2], k.data_ptr(), k.shape[2], n_ctx,
        _ptr(rep_idx), unit_repr.data_ptr(), block_qsum.data_ptr(), wp, wb, _stream(stream, k)))


def infllm_score_units_qsum(cfg, block_qsum, q_pos: int, chunk_len: int, n_chunks: int, unit_repr,
                            scores, stream=None) -> None:
    """Chunk scores with the chunk query sums taken from block query sums."""
    _check(block_qsum, "block_qsum", torch.float64, 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    _check(scores, "scores", torch.float32, 4)
    batch, U = block_qsum.shape[0], unit_repr.shape[2]
    if tuple(scores.shape) != (batch, cfg.n_kv_heads, n_chunks, U):
        raise ValueError("scores must be [batch, H_kv, n_chunks, U]")
    _raise("infllm_score_units_qsum", lib().infllm_score_units_qsum(
        ctypes.byref(cfg), batch, block_qsum.data_ptr(), block_qsum.shape[2], q_pos, chunk_len,
        n_chunks, unit_repr.data_ptr(), U, scores.data_ptr(), _stream(stream, scores)))


def infllm_build_units_range(cfg, q, k, n_ctx: int, u_begin: int, u_end: int, rep_idx, unit_repr,
                             ws=None, stream=None) -> None:
    """Rows u_begin .. u_end-1 of a unit pool [batch, H_kv, pool_units, .]."""
    dt = _dtype_of(cfg)
    if cfg.rep_mode == INFLLM_REP_TOKENS:
        _check(q, "q", dt, 4)
        _check(rep_idx, "rep_idx", torch.int32, 4)
    _check(k, "k", dt, 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    batch, pool = k.shape[0], unit_repr.shape[2]
    if tuple(unit_repr.shape) != (batch, cfg.n_kv_heads, pool, cfg.head_dim):
        raise ValueError("unit_repr must be [batch, H_kv, pool_units, d]")
    if rep_idx is not None and tuple(rep_idx.shape) != (batch, cfg.n_kv_heads, pool, cfg.rep_k):
        raise ValueError("rep_idx must be [batch, H_kv, pool_units, r_k]")
    q_cap = q.shape[2] if q is not None else 0
    wp, wb = _ws(ws)
    _raise("infllm_build_units_range", lib().infllm_build_units_range(
        ctypes.byref(cfg), batch, _ptr(q), q_cap, k.data_ptr(), k.shape[2], n_ctx, u_begin, u_end,
        pool, _ptr(rep_idx), unit_repr.data_ptr(), wp, wb, _stream(stream, k)))


def infllm_score_units(cfg, q, q_off: int, q_pos: int, chunk_len: int, n_chunks: int, unit_repr,
                       scores, ws=None, stream=None) -> None:
    _check(q, "q", _dtype_of(cfg), 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    _check(scores, "scores", torch.float32, 4)
    batch, U = q.shape[0], unit_repr.shape[2]
    if tuple(scores.shape) != (batch, cfg.n_kv_heads, n_chunks, U):
        raise ValueError("scores must be [batch, H_kv, n_chunks, U]")
    wp, wb = _ws(ws)
    _raise("infllm_score_units", lib().infllm_score_units(
        ctypes.byref(cfg), batch, q.data_ptr(), q.shape[2], q_off, q_pos, chunk_len, n_chunks,
        unit_repr.data_ptr(), U, scores.data_ptr(), wp, wb, _stream(stream, q)))


def _check_pos(pos, batch):
    _check(pos, "pos", torch.int64, 1)
    if pos.shape[0] != batch:
        raise ValueError("pos must be [batch] int64")


def infllm_score_units_varlen(cfg, q, q_off: int, pos, chunk_len: int, n_chunks: int, unit_repr,
                              scores, ws=None, stream=None) -> None:
    """pos: device int64 [batch], the position of row q_off per sequence."""
    _check(q, "q", _dtype_of(cfg), 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    _check(scores, "scores", torch.float32, 4)
    batch, U = q.shape[0], unit_repr.shape[2]
    _check_pos(pos, batch)
    if tuple(scores.shape) != (batch, cfg.n_kv_heads, n_chunks, U):
        raise ValueError("scores must be [batch, H_kv, n_chunks, U]")
    wp, wb = _ws(ws)
    _raise("infllm_score_units_varlen", lib().infllm_score_units_varlen(
        ctypes.byref(cfg), batch, q.data_ptr(), q.shape[2], q_off, pos.data_ptr(), chunk_len,
        n_chunks, unit_repr.data_ptr(), U, scores.data_ptr(), wp, wb, _stream(stream, q)))


def infllm_select_units(cfg, q, q_off: int, q_pos: int, chunk_len: int, n_chunks: int, unit_repr,
                        scores, sel, pos=None, ws=None, stream=None) -> None:
    """Scores and top-k in one call; pos (device int64 [batch]) replaces q_pos
    when given."""
    _check(q, "q", _dtype_of(cfg), 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    _check(scores, "scores", torch.float32, 4)
    _check(sel, "sel", torch.int32, 4)
    batch, U = q.shape[0], unit_repr.shape[2]
    if pos is not None:
        _check_pos(pos, batch)
    if tuple(scores.shape) != (batch, cfg.n_kv_heads, n_chunks, U):
        raise ValueError("scores must be [batch, H_kv, n_chunks, U]")
    if tuple(sel.shape) != (batch, cfg.n_kv_heads, n_chunks, cfg.top_k):
        raise ValueError("sel must be [batch, H_kv, n_chunks, k_m]")
    wp, wb = _ws(ws)
    _raise("infllm_select_units", lib().infllm_select_units(
        ctypes.byref(cfg), batch, q.data_ptr(), q.shape[2], q_off, q_pos, _ptr(pos), chunk_len,
        n_chunks, unit_repr.data_ptr(), U, scores.data_ptr(), sel.data_ptr(), wp, wb,
        _stream(stream, q)))


def infllm_topk_units(cfg, scores, sel, ws=None, stream=None) -> None:
    _check(scores, "scores", torch.float32, 4)
    _check(sel, "sel", torch.int32, 4)
    batch, _, n_chunks, U = scores.shape
    if tuple(sel.shape) != (batch, cfg.n_kv_heads, n_chunks, cfg.top_k):
        raise ValueError("sel must be [batch, H_kv, n_chunks, k_m]")
    wp, wb = _ws(ws)
    _raise("infllm_topk_units", lib().infllm_topk_units(
        ctypes.byref(cfg), batch, n_chunks, scores.data_ptr(), U, sel.data_ptr(), wp, wb,
        _stream(stream, scores)))


def infllm_attend(cfg, q, q_off: int, q_pos: int, chunk_len: int, n_chunks: int, k, v, sel, out,
                  lse=None, out_off: int = 0, ws=None, stream=None) -> None:
    dt = _dtype_of(cfg)
    _check(q, "q", dt, 4)
    _check(k, "k", dt, 4)
    _check(v, "v", dt, 4)
    _check(out, "out", dt, 4)
    if sel is not None:
        _check(sel, "sel", torch.int32, 4)
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    wp, wb = _ws(ws)
    _raise("infllm_attend", lib().infllm_attend(
        ctypes.byref(cfg), q.shape[0], q.data_ptr(), q.shape[2], q_off, q_pos, chunk_len, n_chunks,
        k.data_ptr(), v.data_ptr(), k.shape[2], _ptr(sel), out.data_ptr(), _ptr(lse),
        out.shape[2], out_off, wp, wb, _stream(stream, q)))


def infllm_attend_varlen(cfg, q, q_off: int, pos, chunk_len: int, n_chunks: int, k, v, sel, out,
                         lse=None, out_off: int = 0, ws=None, stream=None) -> None:
    """pos: device int64 [batch], the position of row q_off per sequence."""
    dt = _dtype_of(cfg)
    _check(q, "q", dt, 4)
    _check(k, "k", dt, 4)
    _check(v, "v", dt, 4)
    _check(out, "out", dt, 4)
    _check_pos(pos, q.shape[0])
    if sel is not None:
        _check(sel, "sel", torch.int32, 4)
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    wp, wb = _ws(ws)
    _raise("infllm_attend_varlen", lib().infllm_attend_varlen(
        ctypes.byref(cfg), q.shape[0], q.data_ptr(), q.shape[2], q_off, pos.data_ptr(), chunk_len,
        n_chunks, k.data_ptr(), v.data_ptr(), k.shape[2], _ptr(sel), out.data_ptr(), _ptr(lse),
        out.shape[2], out_off, wp, wb, _stream(stream, q)))


def infllm_select_attend(cfg, q, q_off: int, q_pos: int, n_pos: int, unit_repr, k, v, scores, sel,
                         out, lse=None, out_off: int = 0, pos=None, ws=None, stream=None) -> None:
    """One decode step for n_pos single-query positions: scores, top-k and
    attention (one launch where the shapes allow); pos (device int64
    [batch]) replaces q_pos when given."""
    dt = _dtype_of(cfg)
    _check(q, "q", dt, 4)
    _check(k, "k", dt, 4)
    _check(v, "v", dt, 4)
    _check(out, "out", dt, 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    _check(scores, "scores", torch.float32, 4)
    _check(sel, "sel", torch.int32, 4)
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    batch, U = q.shape[0], unit_repr.shape[2]
    if pos is not None:
        _check_pos(pos, batch)
    if tuple(scores.shape) != (batch, cfg.n_kv_heads, n_pos, U):
        raise ValueError("scores must be [batch, H_kv, n_pos, U]")
    if tuple(sel.shape) != (batch, cfg.n_kv_heads, n_pos, cfg.top_k):
        raise ValueError("sel must be [batch, H_kv, n_pos, k_m]")
    wp, wb = _ws(ws)
    _raise("infllm_select_attend", lib().infllm_select_attend(
        ctypes.byref(cfg), batch, q.data_ptr(), q.shape[2], q_off, q_pos, _ptr(pos), n_pos,
        unit_repr.data_ptr(), U, k.data_ptr(), v.data_ptr(), k.shape[2], scores.data_ptr(),
        sel.data_ptr(), out.data_ptr(), _ptr(lse), out.shape[2], out_off, wp, wb,
        _stream(stream, q)))


def infllm_select_attend_static(cfg, q, q_off: int, q_pos: int, n_pos: int, unit_repr, k, v, scores,
                                sel, out, lse=None, out_off: int = 0, pos=None,
                                stream=None) -> None:
    """infllm_select_attend on the library's own scratch memory (no workspace:
    nothing is allocated)."""
    dt = _dtype_of(cfg)
    _check(q, "q", dt, 4)
    _check(k, "k", dt, 4)
    _check(v, "v", dt, 4)
    _check(out, "out", dt, 4)
    _check(unit_repr, "unit_repr", torch.float32, 4)
    _check(scores, "scores", torch.float32, 4)
    _check(sel, "sel", torch.int32, 4)
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    batch, U = q.shape[0], unit_repr.shape[2]
    if pos is not None:
        _check_pos(pos, batch)
    if tuple(scores.shape) != (batch, cfg.n_kv_heads, n_pos, U):
        raise ValueError("scores must be [batch, H_kv, n_pos, U]")
    if tuple(sel.shape) != (batch, cfg.n_kv_heads, n_pos, cfg.top_k):
        raise ValueError("sel must be [batch, H_kv, n_pos, k_m]")
    _raise("infllm_select_attend_static", lib().infllm_select_attend_static(
        ctypes.byref(cfg), batch, q.data_ptr(), q.shape[2], q_off, q_pos, _ptr(pos), n_pos,
        unit_repr.data_ptr(), U, k.data_ptr(), v.data_ptr(), k.shape[2], scores.data_ptr(),
        sel.data_ptr(), out.data_ptr(), _ptr(lse), out.shape[2], out_off, _stream(stream, q)))


# ------------------------------------------------------------------ unit cache
def infllm_cache_state_size(cfg: infllm_config, batch: int, n_units: int, n_slots: int) -> int:
    return int(lib().infllm_cache_state_size(ctypes.byref(cfg), batch, n_units, n_slots))


def cache_state(cfg: infllm_config, batch: int, n_units: int, n_slots: int,
                device="cuda") -> torch.Tensor:
    """A zero-filled (empty) unit cache state."""
    size = infllm_cache_state_size(cfg, batch, n_units, n_slots)
    if size == 0:
        raise ValueError("invalid unit cache shape")
    return torch.zeros(size, dtype=torch.uint8, device=device)


def _check_host(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor) or t.is_cuda or t.dtype != dtype or t.dim() != 4 \
            or not t.is_contiguous() or not t.is_pinned():
        raise ValueError("%s must be a contiguous 4D %s tensor in pinned host memory" %
                         (name, dtype))


def infllm_cache_fetch(cfg, sel, n_units: int, step: int, k_host, v_host, cache_k, cache_v, state,
                       stream=None) -> None:
    """sel [b, H_kv, n_pos, k_m] (device); k_host / v_host [b, H_kv, host_cap, d] pinned;
    cache_k / cache_v [b, H_kv, n_slots, B, d] (device)."""
    dt = _dtype_of(cfg)
    _check(sel, "sel", torch.int32, 4)
    _check_host(k_host, "k_host", dt)
    _check_host(v_host, "v_host", dt)
    _check(cache_k, "cache_k", dt, 5)
    _check(cache_v, "cache_v", dt, 5)
    if k_host.shape != v_host.shape or cache_k.shape != cache_v.shape:
        raise ValueError("K and V buffers must have the same shapes")
    b, _, n_pos, _ = sel.shape
    _raise("infllm_cache_fetch", lib().infllm_cache_fetch(
        ctypes.byref(cfg), b, n_pos, sel.data_ptr(), n_units, step, k_host.data_ptr(),
        v_host.data_ptr(), k_host.shape[2], cache_k.data_ptr(), cache_v.data_ptr(),
        cache_k.shape[2], state.data_ptr(), _stream(stream, sel)))


def infllm_attend_cached(cfg, q, q_off: int, q_pos: int, n_pos: int, k_local, v_local,
                         ctx_cap: int, sel, n_units: int, cache_k, cache_v, state, out, lse=None,
                         out_off: int = 0, pos=None, ws=None, stream=None) -> None:
    """Decode attention (n_pos single positions) with units' keys from the cache;
    k_local / v_local [b, H_kv, local_cap, d]: initial tokens, then a ring."""
    dt = _dtype_of(cfg)
    _check(q, "q", dt, 4)
    _check(k_local, "k_local", dt, 4)
    _check(v_local, "v_local", dt, 4)
    _check(out, "out", dt, 4)
    _check(cache_k, "cache_k", dt, 5)
    _check(cache_v, "cache_v", dt, 5)
    if sel is not None:
        _check(sel, "sel", torch.int32, 4)
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
    if pos is not None:
        _check_pos(pos, q.shape[0])
    wp, wb = _ws(ws)
    _raise("infllm_attend_cached", lib().infllm_attend_cached(
        ctypes.byref(cfg), q.shape[0], q.data_ptr(), q.shape[2], q_off, q_pos, _ptr(pos), n_pos,
        k_local.data_ptr(), v_local.data_ptr(), k_local.shape[2], ctx_cap, _ptr(sel), n_units,
        cache_k.data_ptr(), cache_v.data_ptr(), cache_k.shape[2], state.data_ptr(),
        out.data_ptr(), _ptr(lse), out.shape[2], out_off, wp, wb, _stream(stream, q)))


def infllm_cache_stats(state: torch.Tensor, stream=None) -> tuple[int, int]:
    """(hits, misses) since the state was zero-filled (synchronises)."""
    h, m = _i64(0), _i64(0)
    _raise("infllm_cache_stats", lib().infllm_cache_stats(
        state.data_ptr(), ctypes.byref(h), ctypes.byref(m), _stream(stream, state)))
    return int(h.value), int(m.value)
