"""Python binding of libspecverify, the speculative-decoding verify step on
AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the verify runs in the library's HIP
kernels. Tensors are taken as device-memory handles; the call is enqueued on
the tensor device's current torch stream. The functions carry the C ABI's
names (``sv_softmax_warp``, ``sv_verify_greedy``, ``sv_accept``; see
``include/specverify.h``). ``verify_greedy`` and ``accept`` add the
single-sequence forms of the spec-verify card's API ("API" section):
``(n_accepted, next_token)`` for one ``[K+1, V]`` target.

There is no fallback: if the library is not built, importing this package
raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch  # loads the HIP runtime first, so the library binds to the same one

__all__ = ["sv_softmax_warp", "sv_softmax_warp_workspace_bytes", "sv_softmax_warp_noalloc",
           "SV_NOALLOC_SCRATCH_BYTES", "sv_set_wait_limit", "sv_set_greedy_lookahead", "SV_GREEDY_LOOKAHEAD",
           "sv_verify_greedy",
           "sv_verify_greedy_workspace_bytes", "sv_accept",
           "sv_accept_logits", "sv_accept_logits_workspace_bytes", "sv_softmax_warp_filtered", "sv_verify_greedy_margin", "sv_gate_update",
           "sv_gate_choose", "GATE_DEFAULTS", "sv_commit", "SpeculativeDecoder", "sv_apply_penalties",
           "sv_apply_penalties_workspace_bytes",
           "verify_greedy", "accept", "library_path",
           "SV_F32", "SV_BF16", "SV_MAX_K", "SpecVerifyError", "abi_version"]

SV_F32, SV_BF16 = 0, 1


class Penalties(ctypes.Structure):
    """sv_penalties of include/specverify.h (device pointers, host struct)."""
    _fields_ = [("seq", ctypes.c_void_p), ("seq_len", ctypes.c_void_p), ("cap", ctypes.c_int32),
                ("draft_tokens", ctypes.c_void_p), ("K", ctypes.c_int32), ("repetition", ctypes.c_void_p),
                ("presence", ctypes.c_void_p), ("frequency", ctypes.c_void_p)]


class GateParams(ctypes.Structure):
    """sv_gate_params of include/specverify.h."""
    _fields_ = [("draft_ms", ctypes.c_double), ("verify_base_ms", ctypes.c_double),
                ("verify_slope_ms", ctypes.c_double), ("plain_ms", ctypes.c_double), ("margin", ctypes.c_double),
                ("min_draft", ctypes.c_int32), ("margin_threshold", ctypes.c_float)]
SV_MAX_K = 64
_STATUS = {0: "SV_OK", 1: "SV_ERR_INVALID_ARG", 2: "SV_ERR_UNSUPPORTED", 3: "SV_ERR_HIP", 4: "SV_ERR_WORKSPACE"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libspecverify.so")


class SpecVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {detail}")
        self.status = status


def _load():
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"libspecverify is not built ({path} missing); run __graft_entry__.build() or "
                          f"python draft_token_verification_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i32, i64, c_int = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
    lib.sv_abi_version.restype = c_int
    lib.sv_status_string.argtypes = [c_int]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_last_error.restype = ctypes.c_char_p
    lib.sv_softmax_warp.argtypes = [vp, c_int, i32, i32, i64, vp, i32, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
    lib.sv_softmax_warp_workspace_bytes.argtypes = [i32, i32, i64]
    lib.sv_softmax_warp_noalloc.argtypes = [vp, c_int, i32, i32, i64, vp, i32, ctypes.c_float, vp, vp]
    lib.sv_softmax_warp_noalloc.restype = c_int
    lib.sv_verify_greedy_margin.argtypes = [vp, c_int, i32, i32, i64, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sv_verify_greedy_margin.restype = c_int
    lib.sv_gate_update.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, ctypes.c_double, vp]
    lib.sv_gate_update.restype = c_int
    lib.sv_gate_choose.argtypes = [vp, vp, i32, i32, i32, vp, vp, ctypes.POINTER(GateParams), vp, vp]
    lib.sv_gate_choose.restype = c_int
    lib.sv_commit.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, i32, vp]
    lib.sv_commit.restype = c_int
    lib.sv_apply_penalties.argtypes = [vp, c_int, i32, i32, i64, vp, i32, ctypes.POINTER(Penalties), vp, vp,
                                       ctypes.c_size_t, vp]
    lib.sv_apply_penalties.restype = c_int
    lib.sv_apply_penalties_workspace_bytes.argtypes = [i32, i32]
    lib.sv_apply_penalties_workspace_bytes.restype = ctypes.c_size_t
    lib.sv_softmax_warp_filtered.argtypes = [vp, c_int, i32, i32, i64, vp, i32, ctypes.c_float, vp, vp, vp, vp]
    lib.sv_softmax_warp_filtered.restype = c_int
    lib.sv_softmax_warp_workspace_bytes.restype = ctypes.c_size_t
    lib.sv_set_wait_limit.argtypes = [i32]
    lib.sv_set_wait_limit.restype = c_int
    lib.sv_set_greedy_lookahead.argtypes = [i32]
    lib.sv_set_greedy_lookahead.restype = c_int
    lib.sv_softmax_warp.restype = c_int
    lib.sv_verify_greedy.argtypes = [vp, c_int, i32, i32, i64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sv_verify_greedy_workspace_bytes.argtypes = [i32, i32, i64]
    lib.sv_verify_greedy_workspace_bytes.restype = ctypes.c_size_t
    lib.sv_verify_greedy.restype = c_int
    lib.sv_accept.argtypes = [vp, vp, i32, i32, i64, vp, vp, vp, vp, vp, vp]
    lib.sv_accept.restype = c_int
    lib.sv_accept_logits.argtypes = [vp, vp, c_int, i32, i32, i64, ctypes.c_float, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    lib.sv_accept_logits_workspace_bytes.argtypes = [i32, i32, i64]
    lib.sv_accept_logits_workspace_bytes.restype = ctypes.c_size_t
    lib.sv_accept_logits.restype = c_int
    lib.sv_accept_logits_lse.argtypes = [vp, vp, c_int, i32, i32, i64, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
    lib.sv_accept_logits_lse.restype = c_int
    if lib.sv_abi_version() != 4:
        raise ImportError("libspecverify ABI version mismatch")
    return lib


_lib = _load()


def abi_version() -> int:
    return int(_lib.sv_abi_version())


def _check(fn: str, status: int):
    if status != 0:
        raise SpecVerifyError(fn, status, _lib.sv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, what: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _int32(t: Optional[torch.Tensor], what: str, device) -> Optional[torch.Tensor]:
    if t is None:
        return None
    _dev(t, what)
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    if t.dtype == torch.int32:
        return t
    if t.dtype == torch.int64:
        return t.to(torch.int32)
    raise TypeError(f"{what} must be int32 (or int64), got {t.dtype}")


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"{what} must be float32 or bfloat16, got {t.dtype}")


def _on(device):
    """The device guard of a call: entered only when `device` is not already the
    current device (switching costs a few microseconds per call)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _out(shape, device, out: Optional[torch.Tensor], dtype, what) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(out, what)
    if out.dtype != dtype or tuple(out.shape) != tuple(shape) or out.device != device:
        raise ValueError(f"{what} must be {dtype} of shape {tuple(shape)} on {device}")
    return out


_WORKSPACES = {}
_RETIRED = []  # superseded workspaces, kept alive for the life of the process


def _workspace(nbytes: int, device, stream, kind: str = "fill") -> Optional[torch.Tensor]:
    """A workspace of at least nbytes, kept per (device, stream) so that calls
    on one stream reuse it and calls on different streams never share one.

    A workspace is never freed: a HIP graph captured earlier holds its raw
    address, and a replay after the buffer went back to the allocator would
    write exchange slots into another tensor's memory. When a call needs more
    bytes, the old buffer is retired (kept alive) and the new one is at least
    twice its size, so a stream keeps O(log(largest size)) buffers.

    ``kind`` "zero" is the greedy verify's workspace, kept apart from the others:
    it must hold zeros before its first use and only the greedy verify may
    write it (every call leaves it zero); the others reset their slots
    themselves at each call."""
    if nbytes == 0:
        return None
    key = (device.index, stream, kind)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _RETIRED.append(ws)
            nbytes = max(nbytes, 2 * ws.numel())
        if kind == "zero":
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        else:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def _workspace_arg(workspace: Optional[torch.Tensor], need: int, device, stream, what: str, kind: str = "fill"):
    """(pointer, bytes) of the caller's workspace, or of the one kept per
    device and stream when none is given."""
    if workspace is None:
        workspace = _workspace(need, device, stream, kind)
    elif workspace.device != device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on the {what}' device")
    return _ptr(workspace), 0 if workspace is None else workspace.numel()


def sv_verify_greedy_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(_lib.sv_verify_greedy_workspace_bytes(B, K, V))


def sv_softmax_warp_workspace_bytes(B: int, R: int, V: int) -> int:
    return int(_lib.sv_softmax_warp_workspace_bytes(B, R, V))


def sv_set_wait_limit(polls: int, device=None) -> None:
    """Diagnostic: polls before a warp workgroup computes its row's statistics alone (0 forces it)."""
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check("sv_set_wait_limit", _lib.sv_set_wait_limit(int(polls)))


SV_GREEDY_LOOKAHEAD = 0


def sv_set_greedy_lookahead(rows: int = SV_GREEDY_LOOKAHEAD) -> None:
    """Rows the split greedy walk reads ahead of its decision, process-wide (0, the default, is the
    exact walk; K + 1 or more reads every live row). Results never change, only bytes read and time."""
    _check("sv_set_greedy_lookahead", _lib.sv_set_greedy_lookahead(int(rows)))


def sv_softmax_warp(logits: torch.Tensor, temperature: float = 1.0, draft_lens: Optional[torch.Tensor] = None,
                    extra_rows: int = 0, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """probs[b, r] = softmax(logits[b, r] / T) for the live rows of logits [B, R, V].

    Live rows are r < clamp(draft_lens[b], 0, R - extra_rows) + extra_rows
    (all rows if draft_lens is None). Returns fp32 [B, R, V]; rows that are not
    live are left as they were in ``out`` (uninitialised if ``out`` is None).
    ``workspace`` (a uint8 device tensor) defaults to one kept per device and
    stream, sized by sv_softmax_warp_workspace_bytes.
    """
    _dev(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must be [B, R, V]")
    B, R, V = logits.shape
    dev = logits.device
    lens = _int32(draft_lens, "draft_lens", dev)
    if lens is not None and tuple(lens.shape) != (B,):
        raise ValueError("draft_lens must be [B]")
    probs = _out((B, R, V), dev, out, torch.float32, "out")
    with _on(dev):
        stream = _stream(dev)
        if workspace is None:
            workspace = _workspace(sv_softmax_warp_workspace_bytes(B, R, V) if B > 0 else 0, dev, stream.value)
        elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the logits' device")
        ws_bytes = 0 if workspace is None else workspace.numel()
        st = _lib.sv_softmax_warp(_ptr(logits), _dtype_code(logits, "logits"), B, R, V, _ptr(lens), int(extra_rows),
                                  float(temperature), _ptr(probs), _ptr(workspace), ws_bytes, stream)
    _check("sv_softmax_warp", st)
    return probs


SV_NOALLOC_SCRATCH_BYTES = 1 << 20


def sv_softmax_warp_noalloc(logits: torch.Tensor, temperature: float, draft_lens: Optional[torch.Tensor],
                            extra_rows: int, out: torch.Tensor) -> torch.Tensor:
    """sv_softmax_warp without a workspace or any allocation: the library's fixed
    per-device scratch array holds the exchange slots. ``out`` (fp32 [B, R, V]) is
    required; calls that overlap in time on one device must not be issued (they
    share the array)."""
    _dev(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must be [B, R, V]")
    B, R, V = logits.shape
    dev = logits.device
    if draft_lens is not None:
        _dev(draft_lens, "draft_lens")
        if draft_lens.dtype != torch.int32 or tuple(draft_lens.shape) != (B,) or draft_lens.device != dev:
            raise ValueError("draft_lens must be int32 [B] on the logits' device")
    probs = _out((B, R, V), dev, out, torch.float32, "out")
    with _on(dev):
        st = _lib.sv_softmax_warp_noalloc(_ptr(logits), _dtype_code(logits, "logits"), B, R, V, _ptr(draft_lens),
                                          int(extra_rows), float(temperature), _ptr(probs), _stream(dev))
    _check("sv_softmax_warp_noalloc", st)
    return probs


def sv_verify_greedy_margin(target: torch.Tensor, draft_tokens: Optional[torch.Tensor],
                            draft_lens: Optional[torch.Tensor] = None,
                            out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                            workspace: Optional[torch.Tensor] = None):
    """Greedy verify plus the top1 - top2 margin of the row next_token comes from
    -> (n_accepted[B], next_token[B], top2_margin[B] fp32). ``workspace`` as in
    sv_verify_greedy."""
    _dev(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    toks = _int32(draft_tokens, "draft_tokens", dev)
    if K > 0 and (toks is None or tuple(toks.shape) != (B, K)):
        raise ValueError(f"draft_tokens must be [B, K] = {(B, K)}")
    lens = _int32(draft_lens, "draft_lens", dev)
    if lens is not None and tuple(lens.shape) != (B,):
        raise ValueError("draft_lens must be [B]")
    n = _out((B,), dev, None if out is None else out[0], torch.int32, "n_accepted")
    nx = _out((B,), dev, None if out is None else out[1], torch.int32, "next_token")
    mg = _out((B,), dev, None if out is None else out[2], torch.float32, "top2_margin")
    with _on(dev):
        stream = _stream(dev)
        ws, ws_bytes = _workspace_arg(workspace, sv_verify_greedy_workspace_bytes(B, K, V) if B > 0 else 0, dev,
                                      stream.value, "target", "zero")
        st = _lib.sv_verify_greedy_margin(_ptr(target), _dtype_code(target, "target"), B, K, V, _ptr(toks), _ptr(lens),
                                          _ptr(n), _ptr(nx), _ptr(mg), ws, ws_bytes, stream)
    _check("sv_verify_greedy_margin", st)
    return n, nx, mg


# The DSpark notes' defaults (milliseconds; only their ratios matter).
GATE_DEFAULTS = dict(draft_ms=196.0, verify_base_ms=300.0, verify_slope_ms=109.0, plain_ms=303.0, margin=1.15,
                     min_draft=0, margin_threshold=0.0)


def _gate_state(hits: torch.Tensor, trials: torch.Tensor):
    for t, name in ((hits, "hits"), (trials, "trials")):
        _dev(t, name)
        if t.dtype != torch.float64 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float64 [B, NB] device tensor")
    if hits.shape != trials.shape or hits.device != trials.device:
        raise ValueError("hits and trials must match")
    return hits.shape


def sv_gate_update(hits: torch.Tensor, trials: torch.Tensor, K: int, draft_lens: Optional[torch.Tensor],
                   n_accepted: torch.Tensor, buckets: Optional[torch.Tensor] = None, decay: float = 0.9) -> None:
    """Record one verify round into the gate's counts (in place, on the device)."""
    B, NB = _gate_state(hits, trials)
    dev = hits.device
    lens = _int32(draft_lens, "draft_lens", dev)
    na = _int32(n_accepted, "n_accepted", dev)
    bk = _int32(buckets, "buckets", dev)
    if na is None or tuple(na.shape) != (B,) or (lens is not None and tuple(lens.shape) != (B,)):
        raise ValueError("n_accepted and draft_lens must be [B]")
    if bk is not None and tuple(bk.shape) != (B, K):
        raise ValueError(f"buckets must be [B, K] = {(B, K)}")
    with _on(dev):
        st = _lib.sv_gate_update(_ptr(hits), _ptr(trials), B, NB, int(K), _ptr(lens), _ptr(na), _ptr(bk),
                                 float(decay), _stream(dev))
    _check("sv_gate_update", st)


def sv_gate_choose(hits: torch.Tensor, trials: torch.Tensor, K: int, buckets: Optional[torch.Tensor] = None,
                   top2_margin: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   **params) -> torch.Tensor:
    """Next draft length [B] int32 from the gate's counts; params default to GATE_DEFAULTS."""
    B, NB = _gate_state(hits, trials)
    dev = hits.device
    P = dict(GATE_DEFAULTS)
    unknown = set(params) - set(P)
    if unknown:
        raise ValueError(f"unknown gate parameters {sorted(unknown)}")
    P.update(params)
    bk = _int32(buckets, "buckets", dev)
    if bk is not None and tuple(bk.shape) != (B, K):
        raise ValueError(f"buckets must be [B, K] = {(B, K)}")
    if top2_margin is not None:
        _dev(top2_margin, "top2_margin")
        if top2_margin.dtype != torch.float32 or tuple(top2_margin.shape) != (B,):
            raise ValueError("top2_margin must be fp32 [B]")
    nl = _out((B,), dev, out, torch.int32, "out")
    gp = GateParams(P["draft_ms"], P["verify_base_ms"], P["verify_slope_ms"], P["plain_ms"], P["margin"],
                    int(P["min_draft"]), P["margin_threshold"])
    with _on(dev):
        st = _lib.sv_gate_choose(_ptr(hits), _ptr(trials), B, NB, int(K), _ptr(bk), _ptr(top2_margin),
                                 ctypes.byref(gp), _ptr(nl), _stream(dev))
    _check("sv_gate_choose", st)
    return nl


def sv_commit(seq: torch.Tensor, seq_len: torch.Tensor, done: torch.Tensor, draft_tokens: Optional[torch.Tensor],
              n_accepted: torch.Tensor, next_token: torch.Tensor, limit: Optional[torch.Tensor] = None,
              eos: Optional[int] = None) -> None:
    """Append draft_tokens[b, :n_accepted[b]] and next_token[b] to seq[b] in place (int32 device tensors:
    seq [B, cap], seq_len / done / n_accepted / next_token / limit [B], draft_tokens [B, K])."""
    for t, name in ((seq, "seq"), (seq_len, "seq_len"), (done, "done"), (n_accepted, "n_accepted"),
                    (next_token, "next_token")):
        _dev(t, name)
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    B, cap = seq.shape
    K = 0 if draft_tokens is None else draft_tokens.shape[1]
    if draft_tokens is not None and (draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous()
                                     or draft_tokens.shape[0] != B):
        raise ValueError("draft_tokens must be contiguous int32 [B, K]")
    if limit is not None and (limit.dtype != torch.int32 or tuple(limit.shape) != (B,)):
        raise ValueError("limit must be int32 [B]")
    with torch.cuda.device(seq.device):
        st = _lib.sv_commit(_ptr(seq), _ptr(seq_len), _ptr(done), B, cap, _ptr(draft_tokens), K, _ptr(n_accepted),
                            _ptr(next_token), _ptr(limit), -1 if eos is None else int(eos), _stream(seq.device))
    _check("sv_commit", st)


def _per_sequence(v, B: int, dtype: torch.dtype, dev: torch.device, name: str) -> Optional[torch.Tensor]:
    """None stays None; a Python number is broadcast to [B]; a tensor must be [B] (moved and cast)."""
    if v is None:
        return None
    if isinstance(v, torch.Tensor):
        if tuple(v.shape) != (B,):
            raise ValueError(f"{name} must be [B] = {(B,)}")
        return v.to(device=dev, dtype=dtype).contiguous()
    return torch.full((B,), v, dtype=dtype, device=dev)


def sv_apply_penalties_workspace_bytes(B: int, cap: int) -> int:
    return int(_lib.sv_apply_penalties_workspace_bytes(B, cap))


def sv_apply_penalties(logits: torch.Tensor, draft_lens: Optional[torch.Tensor] = None, extra_rows: int = 0,
                       seq: Optional[torch.Tensor] = None, seq_len: Optional[torch.Tensor] = None,
                       draft_tokens: Optional[torch.Tensor] = None, repetition=None, presence=None, frequency=None,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Repetition / presence / frequency penalties of the live rows of logits [B, R, V] -> fp32 [B, R, V].

    Row r of sequence b is penalised with the history seq[b, :seq_len[b]] + draft_tokens[b, :r]
    (seq [B, cap] and draft_tokens [B, K] int32 device tensors, either may be None). The
    per-sequence parameters are None (off), a number, or a [B] tensor. Rows that are not live
    are left as they were in ``out``.
    """
    _dev(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must be [B, R, V]")
    B, R, V = logits.shape
    dev = logits.device
    lens = _int32(draft_lens, "draft_lens", dev)
    if lens is not None and tuple(lens.shape) != (B,):
        raise ValueError("draft_lens must be [B]")
    sq = _int32(seq, "seq", dev)
    sl = _int32(seq_len, "seq_len", dev)
    if sq is not None:
        sq = sq.contiguous()
        if sq.dim() != 2 or sq.shape[0] != B:
            raise ValueError("seq must be [B, cap]")
        if sl is None or tuple(sl.shape) != (B,):
            raise ValueError("seq_len must be [B] with seq")
    tk = _int32(draft_tokens, "draft_tokens", dev)
    if tk is not None:
        tk = tk.contiguous()
        if tk.dim() != 2 or tk.shape[0] != B:
            raise ValueError("draft_tokens must be [B, K]")
    params = [_per_sequence(v, B, torch.float32, dev, n) for v, n in
              ((repetition, "repetition"), (presence, "presence"), (frequency, "frequency"))]
    o = _out((B, R, V), dev, out, torch.float32, "out")
    pen = Penalties(None if sq is None else sq.data_ptr(), None if sl is None else sl.data_ptr(),
                    0 if sq is None else sq.shape[1], None if tk is None else tk.data_ptr(),
                    0 if tk is None else tk.shape[1], *[None if t is None else t.data_ptr() for t in params])
    with _on(dev):
        stream = _stream(dev)
        need = sv_apply_penalties_workspace_bytes(B, sq.shape[1]) if (sq is not None and B > 0) else 0
        ws, ws_bytes = _workspace_arg(workspace, need, dev, stream.value, "logits", "penalty")
        st = _lib.sv_apply_penalties(_ptr(logits), _dtype_code(logits, "logits"), B, R, V, _ptr(lens),
                                     int(extra_rows), ctypes.byref(pen), _ptr(o), ws, ws_bytes, stream)
    _check("sv_apply_penalties", st)
    return o


def sv_softmax_warp_filtered(logits: torch.Tensor, temperature: float = 1.0, draft_lens: Optional[torch.Tensor] = None,
                             extra_rows: int = 0, top_k=None, top_p=None,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Temperature -> top-k -> top-p -> renormalise for the live rows of logits [B, R, V].

    ``top_k`` / ``top_p``: None (off), a number for every sequence, or a [B] tensor.
    Filtered-out ids get probability 0. Rows that are not live are left as in ``out``.
    """
    _dev(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must be [B, R, V]")
    B, R, V = logits.shape
    dev = logits.device
    lens = _int32(draft_lens, "draft_lens", dev)
    if lens is not None and tuple(lens.shape) != (B,):
        raise ValueError("draft_lens must be [B]")
    tk = _per_sequence(top_k, B, torch.int32, dev, "top_k")
    tp = _per_sequence(top_p, B, torch.float32, dev, "top_p")
    probs = _out((B, R, V), dev, out, torch.float32, "out")
    with _on(dev):
        st = _lib.sv_softmax_warp_filtered(_ptr(logits), _dtype_code(logits, "logits"), B, R, V, _ptr(lens),
                                           int(extra_rows), float(temperature), _ptr(tk), _ptr(tp), _ptr(probs),
                                           _stream(dev))
    _check("sv_softmax_warp_filtered", st)
    return probs


def sv_verify_greedy(target: torch.Tensor, draft_tokens: Optional[torch.Tensor],
                     draft_lens: Optional[torch.Tensor] = None,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Greedy verify of target [B, K+1, V] (fp32/bf16 logits or probs) -> (n_accepted[B], next_token[B]).

    ``workspace`` (uint8 device tensor) defaults to one kept per device and stream, sized by
    sv_verify_greedy_workspace_bytes; a zero-size one selects one workgroup per sequence. A
    workspace of your own must hold zeros before its first use and serve only the greedy verify
    (every call leaves it zero).
    """
    _dev(target, "target")
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    toks = _int32(draft_tokens, "draft_tokens", dev)
    if K > 0 and (toks is None or tuple(toks.shape) != (B, K)):
        raise ValueError(f"draft_tokens must be [B, K] = {(B, K)}")
    lens = _int32(draft_lens, "draft_lens", dev)
    if lens is not None and tuple(lens.shape) != (B,):
        raise ValueError("draft_lens must be [B]")
    n = _out((B,), dev, None if out is None else out[0], torch.int32, "n_accepted")
    nx = _out((B,), dev, None if out is None else out[1], torch.int32, "next_token")
    with _on(dev):
        stream = _stream(dev)
        ws, ws_bytes = _workspace_arg(workspace, sv_verify_greedy_workspace_bytes(B, K, V) if B > 0 else 0, dev,
                                      stream.value, "target", "zero")
        st = _lib.sv_verify_greedy(_ptr(target), _dtype_code(target, "target"), B, K, V, _ptr(toks), _ptr(lens),
                                   _ptr(n), _ptr(nx), ws, ws_bytes, stream)
    _check("sv_verify_greedy", st)
    return n, nx


def sv_accept(target_probs: torch.Tensor, draft_probs: Optional[torch.Tensor], draft_tokens: Optional[torch.Tensor],
              uniforms: torch.Tensor, draft_lens: Optional[torch.Tensor] = None,
              out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Speculative-sampling verify -> (n_accepted[B], next_token[B]).

    target_probs [B, K+1, V] fp32, draft_probs [B, K, V] fp32, draft_tokens
    [B, K], uniforms [B, K+1] fp32 in [0, 1).
    """
    _dev(target_probs, "target_probs")
    if target_probs.dim() != 3 or target_probs.dtype != torch.float32:
        raise ValueError("target_probs must be fp32 [B, K+1, V]")
    B, K1, V = target_probs.shape
    K = K1 - 1
    dev = target_probs.device
    if K > 0:
        _dev(draft_probs, "draft_probs")
        if draft_probs.dtype != torch.float32 or tuple(draft_probs.shape) != (B, K, V) or draft_probs.device != dev:
            raise ValueError(f"draft_probs must be fp32 {(B, K, V)} on {dev}")
    toks = _int32(draft_tokens, "draft_tokens", dev)
    if K > 0 and (toks is None or tuple(toks.shape) != (B, K)):
        raise ValueError(f"draft_tokens must be [B, K] = {(B, K)}")
    _dev(uniforms, "uniforms")
    if uniforms.dtype != torch.float32 or tuple(uniforms.shape) != (B, K1) or uniforms.device != dev:
        raise ValueError(f"uniforms must be fp32 {(B, K1)} on {dev}")
    lens = _int32(draft_lens, "draft_lens", dev)
    if lens is not None and tuple(lens.shape) != (B,):
        raise ValueError("draft_lens must be [B]")
    n = _out((B,), dev, None if out is None else out[0], torch.int32, "n_accepted")
    nx = _out((B,), dev, None if out is None else out[1], torch.int32, "next_token")
    with _on(dev):
        st = _lib.sv_accept(_ptr(target_probs), _ptr(draft_probs if K > 0 else None), B, K, V, _ptr(toks), _ptr(lens),
                            _ptr(uniforms), _ptr(n), _ptr(nx), _stream(dev))
    _check("sv_accept", st)
    return n, nx


def sv_accept_logits_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(_lib.sv_accept_logits_workspace_bytes(B, K, V))


def sv_accept_logits(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor],
                     draft_tokens: Optional[torch.Tensor], uniforms: torch.Tensor, temperature: float = 1.0,
                     draft_lens: Optional[torch.Tensor] = None,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None,
                     draft_lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Speculative-sampling verify from logits (fp32 or bf16) -> (n_accepted[B], next_token[B]).

    ``workspace`` (uint8 device tensor) defaults to one kept per device and stream, sized by
    sv_accept_logits_workspace_bytes; a zero-size one selects one workgroup per sequence.

    target_logits [B, K+1, V], draft_logits [B, K, V] (same dtype), draft_tokens [B, K],
    uniforms [B, K+1] fp32; the rows are warped with temperature T on the fly.

    ``draft_lse`` (fp32 [B, K], optional) gives each draft row's normaliser
    log sum_x exp(draft_logits / T) (sv_accept_logits_lse): the draft rows are then read
    only at the rejected position.
    """
    _dev(target_logits, "target_logits")
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    code = _dtype_code(target_logits, "target_logits")
    if K > 0:
        _dev(draft_logits, "draft_logits")
        if draft_logits.dtype != target_logits.dtype or tuple(draft_logits.shape) != (B, K, V) \
                or draft_logits.device != dev:
            raise ValueError(f"draft_logits must be {target_logits.dtype} {(B, K, V)} on {dev}")
    toks = _int32(draft_tokens, "draft_tokens", dev)
    if K > 0 and (toks is None or tuple(toks.shape) != (B, K)):
        raise ValueError(f"draft_tokens must be [B, K] = {(B, K)}")
    _dev(uniforms, "uniforms")
    if uniforms.dtype != torch.float32 or tuple(uniforms.shape) != (B, K1) or uniforms.device != dev:
        raise ValueError(f"uniforms must be fp32 {(B, K1)} on {dev}")
    lens = _int32(draft_lens, "draft_lens", dev)
    if lens is not None and tuple(lens.shape) != (B,):
        raise ValueError("draft_lens must be [B]")
    if draft_lse is not None:
        _dev(draft_lse, "draft_lse")
        if draft_lse.dtype != torch.float32 or tuple(draft_lse.shape) != (B, K) or draft_lse.device != dev:
            raise ValueError(f"draft_lse must be fp32 {(B, K)} on {dev}")
    n = _out((B,), dev, None if out is None else out[0], torch.int32, "n_accepted")
    nx = _out((B,), dev, None if out is None else out[1], torch.int32, "next_token")
    with _on(dev):
        stream = _stream(dev)
        if workspace is None:
            need = _lib.sv_accept_logits_workspace_bytes(B, K, V) if B > 0 else 0
            workspace = _workspace(need, dev, stream.value)
        elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the logits' device")
        ws_bytes = 0 if workspace is None else workspace.numel()
        if draft_lse is None:
            fn = "sv_accept_logits"
            st = _lib.sv_accept_logits(_ptr(target_logits), _ptr(draft_logits if K > 0 else None), code, B, K, V,
                                       float(temperature), _ptr(toks), _ptr(lens), _ptr(uniforms), _ptr(n), _ptr(nx),
                                       _ptr(workspace), ws_bytes, stream)
        else:
            fn = "sv_accept_logits_lse"
            lse = draft_lse.contiguous()
            st = _lib.sv_accept_logits_lse(_ptr(target_logits), _ptr(draft_logits if K > 0 else None), code, B, K,
                                           V, float(temperature), _ptr(lse if K > 0 else None), _ptr(toks),
                                           _ptr(lens), _ptr(uniforms), _ptr(n), _ptr(nx), _ptr(workspace), ws_bytes,
                                           stream)
    _check(fn, st)
    return n, nx


def _batched(x: torch.Tensor, dims: int) -> Tuple[torch.Tensor, bool]:
    if x.dim() == dims - 1:
        return x.unsqueeze(0).contiguous(), True
    return x.contiguous(), False


def verify_greedy(target_probs: torch.Tensor, draft_tokens: torch.Tensor):
    """The spec-verify card's greedy op: target_probs [K+1, V], draft_tokens [K] -> (n_accepted, next_token).

    Batched inputs ([B, K+1, V], [B, K]) return device tensors instead of ints.
    """
    t, single = _batched(target_probs, 3)
    d, _ = _batched(draft_tokens, 2)
    n, nx = sv_verify_greedy(t, d)
    if single:
        return int(n[0]), int(nx[0])
    return n, nx


def accept(target_probs: torch.Tensor, draft_probs: torch.Tensor, draft_tokens: torch.Tensor,
           generator: Optional[torch.Generator] = None):
    """The spec-verify card's sampled op: uniforms come from ``generator``.

    Draws uniforms [B, K+1] with ``torch.rand`` on the inputs' device, so a
    fixed generator gives a fixed result, then calls ``sv_accept``.
    """
    p, single = _batched(target_probs, 3)
    q, _ = _batched(draft_probs, 3)
    d, _ = _batched(draft_tokens, 2)
    B, K1, _V = p.shape
    u = torch.rand((B, K1), generator=generator, device=p.device, dtype=torch.float32)
    n, nx = sv_accept(p, q, d, u)
    if single:
        return int(n[0]), int(nx[0])
    return n, nx


from .decoder import SpeculativeDecoder  # noqa: E402  (uses the functions above)
