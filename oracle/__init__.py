"""fp64 CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY: the slow, obviously correct reference the HIP
library is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and
the benchmark's CPU-baseline leg may import it. It shares no code with the HIP
library and imports nothing of it.

The arithmetic lives in ``sv_oracle.c`` (plain C, fp64, left-to-right loops);
this module only marshals numpy / CPU-torch arrays into it. Inputs may be
fp32, fp64 or bf16 (bf16 passed as its raw 16-bit patterns); every value is
widened exactly to binary64 before any arithmetic.

Every function here has its pins in ``tests/test_oracle_*.py``: worked values
printed on the pages, closed forms, brute force on tiny inputs, exact
enumeration of the output law and statistical tests of the acceptance law.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

__all__ = ["warp_row", "softmax_warp", "argmax_row", "verify_greedy", "accept", "accept_logits", "icdf", "mass",
           "overlap", "F32", "BF16", "F64", "FLAG_RATIO", "FLAG_CDF", "FLAG_ZERO_RESIDUAL",
           "FLAG_NO_MASS", "FLAG_TOPP", "warp_row_filtered", "softmax_warp_filtered", "top2_margin", "gate_update",
           "gate_choose", "GATE_DEFAULTS", "penalize_row", "apply_penalties", "library_path",
           "load_library", "set_threads"]

F32, BF16, F64 = 0, 1, 2
FLAG_RATIO, FLAG_CDF, FLAG_ZERO_RESIDUAL, FLAG_NO_MASS, FLAG_TOPP = 1, 2, 4, 8, 16

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()


def library_path() -> str:
    """The oracle build to load: ``liboracle.so`` beside this file, or the build
    named by SV_ORACLE_LIBRARY (the sanitized build the pins also run on)."""
    return os.environ.get("SV_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")


def load_library(path: str):
    """Load an oracle build at ``path`` and declare its entry points."""
    lib = ctypes.CDLL(path)
    vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.or_warp_row.argtypes = [vp, ctypes.c_int, i64, f64, vp]
    lib.or_softmax_warp.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i32, f64, vp]
    lib.or_warp_row_filtered.argtypes = [vp, ctypes.c_int, i64, f64, i32, f64, f64, vp, ctypes.POINTER(ctypes.c_int32)]
    lib.or_softmax_warp_filtered.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i32, f64, vp, vp, f64, vp, vp]
    lib.or_argmax_row.argtypes = [vp, ctypes.c_int, i64]
    lib.or_argmax_row.restype = i64
    lib.or_verify_greedy.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp]
    lib.or_mass.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, i64]
    lib.or_mass.restype = f64
    lib.or_icdf.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, i64, f64, f64, ctypes.POINTER(ctypes.c_int32)]
    lib.or_icdf.restype = i64
    lib.or_accept.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, ctypes.c_int, f64, vp, vp, vp]
    lib.or_accept_logits.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, f64, vp, vp, vp, ctypes.c_int, f64, vp, vp,
                                     vp]
    lib.or_accept_logits_lse.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, f64, vp, vp, vp, vp, ctypes.c_int, f64,
                                         vp, vp, vp]
    f32 = ctypes.c_float
    lib.or_penalize_row.argtypes = [vp, ctypes.c_int, i64, vp, i64, f32, f32, f32, vp]
    lib.or_apply_penalties.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i32, vp, vp, i64, vp, i64, vp, vp, vp, vp]
    lib.or_top2_margin.argtypes = [vp, ctypes.c_int, i64]
    lib.or_top2_margin.restype = f64
    lib.or_gate_update.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, f64]
    lib.or_gate_choose.argtypes = [vp, vp, i64, i64, i64, vp, vp, f64, f64, f64, f64, f64, i32, f64, vp]
    lib.or_overlap.argtypes = [vp, vp, ctypes.c_int, i64]
    lib.or_overlap.restype = f64
    lib.or_set_threads.argtypes = [ctypes.c_int]
    lib.or_set_threads.restype = ctypes.c_int
    assert lib.or_abi_version() == 1
    return lib


def set_threads(n: int) -> int:
    """Threads the oracle's row loops use from now on; returns the count in effect (timing only)."""
    return int(_lib().or_set_threads(int(n)))


def _lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(library_path()):
                from . import build as _build
                _build.build()
            _LIB = load_library(library_path())
    return _LIB


def _array(x):
    """(contiguous numpy array, dtype code) for a numpy array or CPU torch tensor."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must be host tensors")
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16)), BF16
            x = x.contiguous().numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def _i32(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def warp_row(z, T: float = 1.0, lib=None) -> np.ndarray:
    """softmax(z / T) of one row, fp64."""
    a, dt = _array(z)
    out = np.empty(a.shape[-1], dtype=np.float64)
    (lib or _lib()).or_warp_row(_ptr(a), dt, a.shape[-1], float(T), _ptr(out))
    return out


def softmax_warp(logits, lens=None, extra_rows: int = 0, T: float = 1.0, lib=None) -> np.ndarray:
    """Warp rows r < clamp(lens[b], 0, R - extra_rows) + extra_rows of logits [B, R, V].

    Rows that are not live are left as NaN in the fp64 result.
    """
    a, dt = _array(logits)
    B, R, V = a.shape
    out = np.full((B, R, V), np.nan, dtype=np.float64)
    ln = _i32(lens)
    (lib or _lib()).or_softmax_warp(_ptr(a), dt, B, R, V, _ptr(ln), int(extra_rows), float(T), _ptr(out))
    return out


def warp_row_filtered(z, T: float = 1.0, top_k: int = 0, top_p: float = 1.0, window: float = 1e-5, lib=None):
    """Temperature, top-k, top-p, renormalise (fp64) -> (probabilities, flag)."""
    a, dt = _array(z)
    out = np.empty(a.shape[-1], dtype=np.float64)
    fl = ctypes.c_int32(0)
    (lib or _lib()).or_warp_row_filtered(_ptr(a), dt, a.shape[-1], float(T), int(top_k), float(top_p), float(window),
                                         _ptr(out), ctypes.byref(fl))
    return out, int(fl.value)


def softmax_warp_filtered(logits, lens=None, extra_rows: int = 0, T: float = 1.0, top_k=None, top_p=None,
                          window: float = 1e-5, lib=None):
    """Filtered warp of the live rows of logits [B, R, V] with per-sequence top_k [B] and
    top_p [B] (None: off) -> (probs [B, R, V] fp64 with NaN in dead rows, flags [B, R])."""
    a, dt = _array(logits)
    B, R, V = a.shape
    out = np.full((B, R, V), np.nan, dtype=np.float64)
    flags = np.zeros((B, R), dtype=np.int32)
    ln = _i32(lens)
    tk = _i32(top_k)
    tp = None if top_p is None else np.ascontiguousarray(np.asarray(
        top_p.detach().cpu().numpy() if hasattr(top_p, "detach") else top_p, dtype=np.float32))
    (lib or _lib()).or_softmax_warp_filtered(_ptr(a), dt, B, R, V, _ptr(ln), int(extra_rows), float(T), _ptr(tk),
                                             _ptr(tp), float(window), _ptr(out), _ptr(flags))
    return out, flags


def penalize_row(z, history, theta: float = 1.0, presence: float = 0.0, frequency: float = 0.0, lib=None):
    """Repetition, presence and frequency penalties of one logit row given its token history -> fp32 row."""
    a, dt = _array(z)
    h = _i32(history)
    h = np.zeros(0, np.int32) if h is None else h.ravel()
    out = np.empty(a.shape[-1], dtype=np.float32)
    (lib or _lib()).or_penalize_row(_ptr(a), dt, a.shape[-1], _ptr(h), h.size, float(theta), float(presence),
                                    float(frequency), _ptr(out))
    return out


def _f32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def apply_penalties(logits, lens=None, extra_rows: int = 0, seq=None, seq_len=None, tokens=None, theta=None,
                    presence=None, frequency=None, lib=None):
    """Penalties of the live rows of logits [B, R, V]: row r of sequence b takes the history
    seq[b, :seq_len[b]] + tokens[b, :r]. Per-sequence theta / presence / frequency: None (off), a
    number for every sequence, or [B].
    Returns fp32 [B, R, V] with NaN in rows that are not live."""
    a, dt = _array(logits)
    B, R, V = a.shape
    out = np.full((B, R, V), np.nan, dtype=np.float32)
    ln = _i32(lens)
    sq = _i32(seq)
    sl = _i32(seq_len)
    tk = _i32(tokens)
    cap = 0 if sq is None else sq.shape[1]
    K = 0 if tk is None else tk.shape[1]

    def per_sequence(x, name):  # None, a number for every sequence, or [B]
        if x is None:
            return None
        if np.ndim(x.detach().cpu().numpy() if hasattr(x, "detach") else x) == 0:
            return np.full(B, float(x), dtype=np.float32)
        x = _f32(x)
        if x.shape != (B,):
            raise ValueError(f"{name} must be a number or [B] = {(B,)}")
        return x
    th, pr, fr = (per_sequence(x, n) for x, n in ((theta, "theta"), (presence, "presence"), (frequency, "frequency")))
    (lib or _lib()).or_apply_penalties(_ptr(a), dt, B, R, V, _ptr(ln), int(extra_rows), _ptr(sq), _ptr(sl), cap,
                                       _ptr(tk), K, _ptr(th), _ptr(pr), _ptr(fr), _ptr(out))
    return out


def top2_margin(row, lib=None) -> float:
    """Largest value minus the largest of the others (fp64; +inf for one element)."""
    a, dt = _array(row)
    return float((lib or _lib()).or_top2_margin(_ptr(a), dt, a.shape[-1]))


# the DSpark notes' default gate parameters (draft, verify base and slope, plain decode in ms)
GATE_DEFAULTS = dict(draft_ms=196.0, verify_base_ms=300.0, verify_slope_ms=109.0, plain_ms=303.0, margin=1.15,
                     decay=0.9, min_draft=0, margin_threshold=0.0)


def gate_update(hits, trials, K: int, lens, n_accepted, buckets=None, decay: float = 0.9, lib=None):
    """Record one verify round (draft lens [B] of at most K, n_accepted [B], buckets [B, K] or None
    for the position) into hits / trials [B, NB] (float64 numpy arrays, updated in place)."""
    assert hits.dtype == np.float64 and trials.dtype == np.float64 and hits.flags.c_contiguous
    assert trials.flags.c_contiguous and trials.shape == hits.shape
    B, NB = hits.shape
    ln = _i32(lens)
    na = _i32(n_accepted)
    bk = _i32(buckets)
    (lib or _lib()).or_gate_update(_ptr(hits), _ptr(trials), B, NB, int(K), _ptr(ln), _ptr(na), _ptr(bk),
                                   float(decay))


def gate_choose(hits, trials, K: int, buckets=None, top2_margin=None, lib=None, **params):
    """Next draft length [B] (int32) from the gate's counts; params default to GATE_DEFAULTS."""
    P = dict(GATE_DEFAULTS)
    P.update(params)
    B, NB = hits.shape
    bk = _i32(buckets)
    tm = None if top2_margin is None else np.ascontiguousarray(np.asarray(top2_margin, dtype=np.float32))
    out = np.empty(B, dtype=np.int32)
    (lib or _lib()).or_gate_choose(_ptr(hits), _ptr(trials), B, NB, int(K), _ptr(bk), _ptr(tm), P["draft_ms"],
                                   P["verify_base_ms"], P["verify_slope_ms"], P["plain_ms"], P["margin"],
                                   int(P["min_draft"]), P["margin_threshold"], _ptr(out))
    return out


def argmax_row(row, lib=None) -> int:
    a, dt = _array(row)
    return int((lib or _lib()).or_argmax_row(_ptr(a), dt, a.shape[-1]))


def verify_greedy(target, tokens, lens=None, lib=None):
    """Greedy verify of target [B, K+1, V] against tokens [B, K] -> (n_accepted[B], next_token[B])."""
    a, dt = _array(target)
    B, K1, V = a.shape
    t = _i32(tokens).reshape(B, K1 - 1)
    ln = _i32(lens)
    n = np.empty(B, dtype=np.int32)
    nx = np.empty(B, dtype=np.int32)
    (lib or _lib()).or_verify_greedy(_ptr(a), dt, B, K1 - 1, V, _ptr(t), _ptr(ln), _ptr(n), _ptr(nx))
    return n, nx


def accept(p, q, tokens, uniforms, lens=None, rel_window: float = 1e-5, lib=None):
    """Speculative-sampling verify -> (n_accepted[B], next_token[B], flags[B]).

    p [B, K+1, V], q [B, K, V] (same dtype), tokens [B, K], uniforms [B, K+1]
    (fp32 or fp64). ``flags`` marks sequences whose decisions lie within
    ``rel_window`` (relative) of a ratio or CDF boundary.
    """
    pa, dt = _array(p)
    qa, dq = _array(q)
    if dq != dt:
        raise TypeError("p and q must share a dtype")
    B, K1, V = pa.shape
    K = K1 - 1
    if qa.shape != (B, K, V):
        raise ValueError(f"q shape {qa.shape} != {(B, K, V)}")
    t = _i32(tokens).reshape(B, K)
    ua, du = _array(uniforms)
    if du == BF16 or ua.size != B * K1:
        raise ValueError("uniforms must be fp32/fp64 [B, K+1]")
    ln = _i32(lens)
    n = np.empty(B, dtype=np.int32)
    nx = np.empty(B, dtype=np.int32)
    fl = np.empty(B, dtype=np.int32)
    (lib or _lib()).or_accept(_ptr(pa), _ptr(qa), dt, B, K, V, _ptr(t), _ptr(ln), _ptr(ua), du, float(rel_window), _ptr(n),
                     _ptr(nx), _ptr(fl))
    return n, nx, fl


def accept_logits(zt, zd, tokens, uniforms, lens=None, T: float = 1.0, rel_window: float = 1e-5, lib=None,
                  draft_lse=None):
    """Sampled verify from logits: or_accept on softmax(z / T) of the examined rows, in fp64.

    zt [B, K+1, V], zd [B, K, V] logits (same dtype). Returns (n_accepted, next_token, flags),
    flagged with the same relative ratio and CDF windows as ``accept``.

    draft_lse [B, K] (fp32): each draft row's distribution given by its
    log-normaliser, q_i(x) = exp(zd_i(x) / T - draft_lse[b, i]) (or_accept_logits_lse).
    """
    ta, dt = _array(zt)
    B, K1, V = ta.shape
    K = K1 - 1
    if zd is None and K == 0:
        zd = np.empty((B, 0, V), dtype=ta.dtype)
    da, dd = _array(zd)
    if dd != dt:
        raise TypeError("target and draft logits must share a dtype")
    if da.shape != (B, K, V):
        raise ValueError(f"draft shape {da.shape} != {(B, K, V)}")
    t = np.zeros((B, 0), dtype=np.int32) if tokens is None and K == 0 else _i32(tokens).reshape(B, K)
    ua, du = _array(uniforms)
    if du == BF16 or ua.size != B * K1:
        raise ValueError("uniforms must be fp32/fp64 [B, K+1]")
    ln = _i32(lens)
    n = np.empty(B, dtype=np.int32)
    nx = np.empty(B, dtype=np.int32)
    fl = np.empty(B, dtype=np.int32)
    if draft_lse is None:
        (lib or _lib()).or_accept_logits(_ptr(ta), _ptr(da), dt, B, K, V, float(T), _ptr(t), _ptr(ln), _ptr(ua), du,
                                         float(rel_window), _ptr(n), _ptr(nx), _ptr(fl))
    else:
        ls = _f32(draft_lse)
        if ls.size != B * K:
            raise ValueError(f"draft_lse must hold B*K = {B * K} values, got {ls.size}")
        (lib or _lib()).or_accept_logits_lse(_ptr(ta), _ptr(da), dt, B, K, V, float(T), _ptr(ls), _ptr(t), _ptr(ln),
                                             _ptr(ua), du, float(rel_window), _ptr(n), _ptr(nx), _ptr(fl))
    return n, nx, fl


def mass(p, q=None, lib=None) -> float:
    """sum_x max(0, p - q) (q given) or sum_x max(0, p) (q None), fp64."""
    pa, dt = _array(p)
    if q is None:
        return float((lib or _lib()).or_mass(_ptr(pa), None, dt, 1, pa.shape[-1]))
    qa, _ = _array(q)
    return float((lib or _lib()).or_mass(_ptr(pa), _ptr(qa), dt, 0, pa.shape[-1]))


def icdf(p, u: float, q=None, rel_window: float = 1e-5, lib=None):
    """Draw from norm(max(0, p - q)) (q given) or norm(max(0, p)) with uniform u -> (id, flag)."""
    pa, dt = _array(p)
    qa = None if q is None else _array(q)[0]
    flag = ctypes.c_int32(0)
    x = (lib or _lib()).or_icdf(_ptr(pa), _ptr(qa), dt, 0 if q is not None else 1, pa.shape[-1], float(u), float(rel_window),
                       ctypes.byref(flag))
    return int(x), int(flag.value)


def overlap(p, q, lib=None) -> float:
    """sum_x min(p(x), q(x)): the per-position acceptance probability."""
    pa, dt = _array(p)
    qa, _ = _array(q)
    return float((lib or _lib()).or_overlap(_ptr(pa), _ptr(qa), dt, pa.shape[-1]))
