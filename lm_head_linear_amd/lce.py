"""Thin Python binding of liblce.so (include/lce.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of liblce.so.  Functions carry the C names; tensors are torch
tensors (device tensors for the device entry points), the stream is torch's
current stream on the tensors' device.  If the library has not been built the
first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblce.so")

OK = 580
BF16, F32, F64, I64, F16, U8 = 1, 2, 3, 4, 5, 6
STATUS = {580: "ok", 581: "empty_dimension", 582: "length_mismatch", 583: "dimension_too_large",
          584: "work_budget_exceeded", 585: "non_finite_scalar", 586: "target_id_out_of_range",
          587: "chunk_exceeds_logit_budget", 588: "unknown_objective", 589: "device_error",
          590: "dtype_mismatch"}
_DT = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32, torch.float64: F64,
       torch.int64: I64, torch.uint8: U8, torch.bool: U8}


class LceError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({STATUS.get(status, 'unknown_status')})")
        self.status = status


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("numel", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class Peak(ctypes.Structure):
    _fields_ = [("chunked_cells", ctypes.c_double), ("materialized_cells", ctypes.c_double),
                ("ratio", ctypes.c_double), ("n_chunks", ctypes.c_int64),
                ("status", ctypes.c_int32)]


NUM_KERNELS = 12
KERNEL_KINDS = {"guard": 0, "fwd_gemm": 1, "fwd_merge": 2, "reduce": 3, "dlogit_gemm": 4,
                "dw_gemm": 5, "dh_gemm": 6, "dh_final": 7, "distill": 8, "bwd_gemm": 9,
                "label_ce": 10, "dlogit_rows": 11}


class TimerSlot(ctypes.Structure):
    _fields_ = [("start", ctypes.POINTER(ctypes.c_void_p)), ("stop", ctypes.POINTER(ctypes.c_void_p)),
                ("capacity", ctypes.c_int32), ("used", ctypes.c_int32)]


class Timers(ctypes.Structure):
    _fields_ = [("slot", TimerSlot * NUM_KERNELS)]


class KernelTimer:
    """Caller-owned HIP events that the timed entry points record around each
    launch of the chosen kernel kinds; elapsed times are read back here."""

    def __init__(self, kinds, capacity: int, device=None):
        self.kinds = list(kinds)
        self.capacity = capacity
        self.struct = Timers()
        self._keep = []
        self.events = {}
        for k in self.kinds:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(capacity)]
            for a, b in ev:          # torch creates the HIP event on first record
                a.record()
                b.record()
            starts = (ctypes.c_void_p * capacity)(*[a.cuda_event for a, _ in ev])
            stops = (ctypes.c_void_p * capacity)(*[b.cuda_event for _, b in ev])
            self._keep += [starts, stops]
            sl = self.struct.slot[KERNEL_KINDS[k]]
            sl.start = ctypes.cast(starts, ctypes.POINTER(ctypes.c_void_p))
            sl.stop = ctypes.cast(stops, ctypes.POINTER(ctypes.c_void_p))
            sl.capacity = capacity
            sl.used = 0
            self.events[k] = ev
        torch.cuda.synchronize()

    def reset(self):
        for k in self.kinds:
            self.struct.slot[KERNEL_KINDS[k]].used = 0

    def used(self, kind) -> int:
        return self.struct.slot[KERNEL_KINDS[kind]].used

    def durations_ms(self, kind):
        """Elapsed time of every recorded launch of `kind` (call after a sync)."""
        n = self.used(kind)
        return [a.elapsed_time(b) for a, b in self.events[kind][:n]]


class Loss(ctypes.Structure):
    _fields_ = [("loss_sum", ctypes.c_double), ("loss_mean", ctypes.c_double),
                ("z_sum", ctypes.c_double), ("z_mean", ctypes.c_double),
                ("n_counted", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def lib():
    """The loaded liblce.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        PT = ctypes.POINTER(Tensor)
        L.lce_status_name.restype = ctypes.c_char_p
        L.lce_status_name.argtypes = [i32]
        L.lce_dims_check.restype = i32
        L.lce_dims_check.argtypes = [i64, i64, i64]
        L.lce_chunk_check.restype = i32
        L.lce_chunk_check.argtypes = [i64, i64]
        L.lce_logit_cells.restype = dbl
        L.lce_logit_cells.argtypes = [i64, i64]
        L.lce_work_fits.restype = i32
        L.lce_work_fits.argtypes = [i64, i64, i64, i64]
        L.lce_peak_cells.restype = i32
        L.lce_peak_cells.argtypes = [i64, i64, i64, ctypes.POINTER(Peak)]
        L.lce_workspace_bytes.restype = i64
        L.lce_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
        L.lce_distill_workspace_bytes.restype = i64
        L.lce_distill_workspace_bytes.argtypes = [i64, i64]
        L.lce_forward_backward_workspace_bytes.restype = i64
        L.lce_forward_backward_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
        L.lce_forward_backward_keeps_logits.restype = i32
        L.lce_forward_backward_keeps_logits.argtypes = [i64, i64, i64, i64, i32]
        L.lce_forward.restype = i32
        L.lce_forward.argtypes = [PT, PT, PT, PT, i64, i64, i64, i64, dbl, PT, PT,
                                  ctypes.POINTER(Loss), vp]
        L.lce_loss_fetch.restype = i32
        L.lce_loss_fetch.argtypes = [PT, ctypes.POINTER(Loss), vp]
        L.lce_backward.restype = i32
        L.lce_backward.argtypes = [PT, PT, PT, PT, PT, i64, i64, i64, i64, dbl, dbl, PT, PT, i32,
                                   PT, vp]
        L.lce_distill_fwd_bwd.restype = i32
        L.lce_distill_fwd_bwd.argtypes = [PT, PT, PT, i64, i64, i32, dbl, dbl, dbl, PT, PT,
                                          ctypes.POINTER(Loss), vp]
        L.lce_distill_fwd_bwd_noalloc.restype = i32
        L.lce_distill_fwd_bwd_noalloc.argtypes = [PT, PT, PT, i64, i64, i32, dbl, dbl, dbl, PT,
                                                  ctypes.POINTER(Loss), vp]
        L.lce_ce_logits_fwd_bwd.restype = i32
        L.lce_ce_logits_fwd_bwd.argtypes = [PT, PT, PT, i64, i64, dbl, dbl, PT, PT,
                                            ctypes.POINTER(Loss), vp]
        L.lce_shard_forward.restype = i32
        L.lce_shard_forward.argtypes = [PT, PT, PT, i64, i64, i64, i64, i64, i64, PT, PT, vp]
        L.lce_shard_merge.restype = i32
        L.lce_shard_merge.argtypes = [PT, i32, PT, i64, PT, PT, ctypes.POINTER(Loss), vp]
        L.lce_shard_backward.restype = i32
        L.lce_shard_backward.argtypes = [PT, PT, PT, PT, PT, i64, i64, i64, i64, i64, i64, dbl,
                                         dbl, PT, PT, i32, PT, vp]
        PTM = ctypes.POINTER(Timers)
        L.lce_forward_backward.restype = i32
        L.lce_forward_backward.argtypes = [PT, PT, PT, PT, i64, i64, i64, i64, dbl, dbl, PT, PT,
                                           PT, i32, PT, ctypes.POINTER(Loss), vp]
        L.lce_forward_backward_timed.restype = i32
        L.lce_forward_backward_timed.argtypes = L.lce_forward_backward.argtypes + [PTM]
        L.lce_forward_timed.restype = i32
        L.lce_forward_timed.argtypes = L.lce_forward.argtypes + [PTM]
        L.lce_backward_timed.restype = i32
        L.lce_backward_timed.argtypes = L.lce_backward.argtypes + [PTM]
        L.lce_distill_fwd_bwd_timed.restype = i32
        L.lce_distill_fwd_bwd_timed.argtypes = L.lce_distill_fwd_bwd.argtypes + [PTM]
        L.lce_ce_logits_fwd_bwd_timed.restype = i32
        L.lce_ce_logits_fwd_bwd_timed.argtypes = L.lce_ce_logits_fwd_bwd.argtypes + [PTM]
        _lib = L
    return _lib


def _t(x: Optional[torch.Tensor]) -> Tensor:
    """Flat descriptor of a contiguous tensor (NULL descriptor for None)."""
    if x is None:
        return Tensor(None, 0, 0)
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return Tensor(x.data_ptr(), x.numel(), _DT.get(x.dtype, 0))


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


# ------------------------------------------------------------- host contract

def lce_status_name(code: int) -> str:
    return lib().lce_status_name(int(code)).decode()


def lce_dims_check(n_tok: int, d_model: int, vocab: int) -> int:
    return lib().lce_dims_check(n_tok, d_model, vocab)


def lce_chunk_check(chunk: int, vocab: int) -> int:
    return lib().lce_chunk_check(chunk, vocab)


def lce_logit_cells(chunk: int, vocab: int) -> float:
    return lib().lce_logit_cells(chunk, vocab)


def lce_work_fits(n: int, d: int, v: int, ceiling: int) -> bool:
    return bool(lib().lce_work_fits(n, d, v, ceiling))


def lce_peak_cells(n_tok: int, vocab: int, chunk: int) -> dict:
    p = Peak()
    lib().lce_peak_cells(n_tok, vocab, chunk, ctypes.byref(p))
    return {"chunked_cells": p.chunked_cells, "materialized_cells": p.materialized_cells,
            "ratio": p.ratio, "n_chunks": p.n_chunks, "status": p.status}


def lce_workspace_bytes(n_tok: int, d_model: int, vocab: int, chunk: int, dtype) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return lib().lce_workspace_bytes(n_tok, d_model, vocab, chunk, dt)


def lce_distill_workspace_bytes(n_tok: int, vocab: int) -> int:
    return lib().lce_distill_workspace_bytes(n_tok, vocab)


def lce_forward_backward_workspace_bytes(n_tok: int, d_model: int, vocab: int, chunk: int,
                                         dtype) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return lib().lce_forward_backward_workspace_bytes(n_tok, d_model, vocab, chunk, dt)


def lce_forward_backward_keeps_logits(n_tok: int, d_model: int, vocab: int, chunk: int,
                                      dtype) -> int:
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return lib().lce_forward_backward_keeps_logits(n_tok, d_model, vocab, chunk, dt)


# ------------------------------------------------------------ device calls

def lce_forward(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, chunk, z_coef,
                lse_out, workspace, stream: Optional[int] = None,
                timer: Optional[KernelTimer] = None, sync: bool = True):
    """Direct call of the C entry point (lce_forward_timed when a timer is
    given).  Returns (status, Loss); with sync=False the call passes a NULL
    out (asynchronous) and returns (status, None): lce_loss_fetch reads the
    scalars later."""
    out = Loss() if sync else None
    args = [_t(hidden), _t(weight), _t(targets), _t(loss_mask)]
    lse_t, ws_t = _t(lse_out), _t(workspace)
    call = [*[ctypes.byref(a) for a in args], n_tok, d_model, vocab, chunk, float(z_coef),
            ctypes.byref(lse_t), ctypes.byref(ws_t), ctypes.byref(out) if sync else None,
            stream if stream is not None else _stream(hidden.device)]
    if timer is None:
        st = lib().lce_forward(*call)
    else:
        st = lib().lce_forward_timed(*call, ctypes.byref(timer.struct))
    return st, out


def lce_loss_fetch(workspace, stream: Optional[int] = None):
    """Scalars of the last lce_forward on `workspace` (synchronizes the
    stream).  Returns (status, Loss)."""
    out = Loss()
    ws_t = _t(workspace)
    st = lib().lce_loss_fetch(ctypes.byref(ws_t), ctypes.byref(out),
                              stream if stream is not None else _stream(workspace.device))
    return st, out


def lce_backward(hidden, weight, targets, loss_mask, lse, n_tok, d_model, vocab, chunk, z_coef,
                 grad_out, d_hidden, d_weight, accumulate_d_weight, workspace,
                 stream: Optional[int] = None, timer: Optional[KernelTimer] = None) -> int:
    """Direct call of the C entry point (lce_backward_timed when a timer is
    given).  Returns the status; the call does not wait for the device, so a
    target out of range shows in the next lce_loss_fetch (586)."""
    ts = [_t(hidden), _t(weight), _t(targets), _t(loss_mask), _t(lse)]
    dh, dw, ws = _t(d_hidden), _t(d_weight), _t(workspace)
    call = [*[ctypes.byref(a) for a in ts], n_tok, d_model, vocab, chunk, float(z_coef),
            float(grad_out), ctypes.byref(dh), ctypes.byref(dw), int(bool(accumulate_d_weight)),
            ctypes.byref(ws), stream if stream is not None else _stream(hidden.device)]
    if timer is None:
        return lib().lce_backward(*call)
    return lib().lce_backward_timed(*call, ctypes.byref(timer.struct))


def lce_distill_fwd_bwd(student, teacher, loss_mask, n_tok, vocab, objective, temperature,
                        z_coef, grad_out, grad_logits, workspace, stream: Optional[int] = None,
                        timer: Optional[KernelTimer] = None, sync: bool = True):
    """Direct call of the C entry point (the _timed variant when a timer is
    given).  Returns (status, Loss or None when sync is False: the call is then
    asynchronous and lce_loss_fetch(workspace) returns the scalars)."""
    out = Loss() if sync else None
    ts = [_t(student), _t(teacher), _t(loss_mask)]
    g, ws = _t(grad_logits), _t(workspace)
    call = [*[ctypes.byref(a) for a in ts], n_tok, vocab, int(objective), float(temperature),
            float(z_coef), float(grad_out), ctypes.byref(g), ctypes.byref(ws),
            ctypes.byref(out) if sync else None,
            stream if stream is not None else _stream(student.device)]
    if timer is None:
        st = lib().lce_distill_fwd_bwd(*call)
    else:
        st = lib().lce_distill_fwd_bwd_timed(*call, ctypes.byref(timer.struct))
    return st, out


def lce_distill_fwd_bwd_noalloc(student, teacher, loss_mask, n_tok, vocab, objective,
                                temperature, z_coef, grad_out, grad_logits,
                                stream: Optional[int] = None):
    """Direct call of the allocation-free C entry point (its scratch is the
    library's static device array).  Returns (status, Loss)."""
    out = Loss()
    ts = [_t(student), _t(teacher), _t(loss_mask)]
    g = _t(grad_logits)
    st = lib().lce_distill_fwd_bwd_noalloc(
        *[ctypes.byref(a) for a in ts], n_tok, vocab, int(objective), float(temperature),
        float(z_coef), float(grad_out), ctypes.byref(g), ctypes.byref(out),
        stream if stream is not None else _stream(student.device))
    return st, out


def lce_ce_logits_fwd_bwd(logits, targets, loss_mask, n_tok, vocab, z_coef, grad_out,
                          grad_logits, workspace, stream: Optional[int] = None,
                          timer: Optional[KernelTimer] = None, sync: bool = True):
    """Direct call of the C entry point (the _timed variant when a timer is
    given); grad_logits None computes the loss only.  Returns (status, Loss or
    None when sync is False: the call is then asynchronous and
    lce_loss_fetch(workspace) returns the scalars, or 586)."""
    out = Loss() if sync else None
    ts = [_t(logits), _t(targets), _t(loss_mask)]
    g, ws = _t(grad_logits), _t(workspace)
    call = [*[ctypes.byref(a) for a in ts], n_tok, vocab, float(z_coef), float(grad_out),
            ctypes.byref(g), ctypes.byref(ws), ctypes.byref(out) if sync else None,
            stream if stream is not None else _stream(logits.device)]
    if timer is None:
        st = lib().lce_ce_logits_fwd_bwd(*call)
    else:
        st = lib().lce_ce_logits_fwd_bwd_timed(*call, ctypes.byref(timer.struct))
    return st, out


def lce_shard_forward(hidden, weight_shard, targets, n_tok, d_model, vocab_shard, vocab_offset,
                      vocab_total, chunk, stats, workspace, stream: Optional[int] = None) -> int:
    """Direct call of the C entry point; returns the status.  The call does not
    wait for the device: a target out of range shows as 586 in
    lce_loss_fetch(workspace)."""
    ts = [_t(hidden), _t(weight_shard), _t(targets)]
    st_t, ws = _t(stats), _t(workspace)
    return lib().lce_shard_forward(*[ctypes.byref(a) for a in ts], n_tok, d_model, vocab_shard,
                                   vocab_offset, vocab_total, chunk, ctypes.byref(st_t),
                                   ctypes.byref(ws),
                                   stream if stream is not None else _stream(hidden.device))


def lce_shard_merge(stats, n_shards, loss_mask, n_tok, lse_out, workspace,
                    stream: Optional[int] = None, sync: bool = True):
    """Direct call of the C entry point.  Returns (status, Loss or None when
    sync is False: the call is then asynchronous and lce_loss_fetch(workspace)
    returns the scalars)."""
    out = Loss() if sync else None
    a, m, l, ws = _t(stats), _t(loss_mask), _t(lse_out), _t(workspace)
    st = lib().lce_shard_merge(ctypes.byref(a), int(n_shards), ctypes.byref(m), n_tok,
                               ctypes.byref(l), ctypes.byref(ws),
                               ctypes.byref(out) if sync else None,
                               stream if stream is not None else _stream(stats.device))
    return st, out


def lce_shard_backward(hidden, weight_shard, targets, loss_mask, lse, n_tok, d_model, vocab_shard,
                       vocab_offset, vocab_total, chunk, z_coef, grad_out, d_hidden_partial,
                       d_weight_shard, accumulate_d_weight, workspace,
                       stream: Optional[int] = None) -> int:
    """Direct call of the C entry point; returns the status."""
    ts = [_t(hidden), _t(weight_shard), _t(targets), _t(loss_mask), _t(lse)]
    dh, dw, ws = _t(d_hidden_partial), _t(d_weight_shard), _t(workspace)
    return lib().lce_shard_backward(*[ctypes.byref(a) for a in ts], n_tok, d_model, vocab_shard,
                                    vocab_offset, vocab_total, chunk, float(z_coef),
                                    float(grad_out), ctypes.byref(dh), ctypes.byref(dw),
                                    int(accumulate_d_weight), ctypes.byref(ws),
                                    stream if stream is not None else _stream(hidden.device))


# ------------------------------------------------- allocating conveniences

def lce_forward_backward(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, chunk,
                         z_coef, grad_out, lse_out, d_hidden, d_weight, accumulate_d_weight,
                         workspace, stream: Optional[int] = None,
                         timer: Optional[KernelTimer] = None, sync: bool = True):
    """Direct call of the C entry point (lce_forward_backward_timed when a
    timer is given).  Returns (status, Loss or None when sync is False)."""
    out = Loss() if sync else None
    ts = [_t(hidden), _t(weight), _t(targets), _t(loss_mask)]
    lse_t, dh, dw, ws = _t(lse_out), _t(d_hidden), _t(d_weight), _t(workspace)
    call = [*[ctypes.byref(a) for a in ts], n_tok, d_model, vocab, chunk, float(z_coef),
            float(grad_out), ctypes.byref(lse_t), ctypes.byref(dh), ctypes.byref(dw),
            int(bool(accumulate_d_weight)), ctypes.byref(ws),
            ctypes.byref(out) if sync else None,
            stream if stream is not None else _stream(hidden.device)]
    if timer is None:
        st = lib().lce_forward_backward(*call)
    else:
        st = lib().lce_forward_backward_timed(*call, ctypes.byref(timer.struct))
    return st, out


def _acc_dtype(dt: torch.dtype) -> torch.dtype:
    return torch.float64 if dt == torch.float64 else torch.float32


def workspace_for(n_tok, d_model, vocab, chunk, dtype, device) -> torch.Tensor:
    nbytes = lce_workspace_bytes(n_tok, d_model, vocab, chunk, dtype)
    if nbytes < 0:
        raise LceError(int(-nbytes), "lce_workspace_bytes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class ForwardResult:
    loss: dict
    lse: torch.Tensor


def forward(hidden, weight, targets, loss_mask=None, chunk=256, z_coef=0.0, workspace=None):
    """Allocate lse and (if needed) the workspace, call lce_forward, raise on refusal."""
    n, D = hidden.shape
    V = weight.shape[0]
    lse = torch.empty(n, dtype=_acc_dtype(hidden.dtype), device=hidden.device)
    ws = workspace if workspace is not None else workspace_for(n, D, V, chunk, hidden.dtype,
                                                               hidden.device)
    st, out = lce_forward(hidden, weight, targets, loss_mask, n, D, V, chunk, z_coef, lse, ws)
    if st != OK:
        raise LceError(st, "lce_forward")
    return ForwardResult(out.as_dict(), lse)


def backward(hidden, weight, targets, lse, loss_mask=None, chunk=256, z_coef=0.0, grad_out=1.0,
             d_weight=None, accumulate=False, workspace=None):
    """Allocate d_hidden (and d_weight unless given), call lce_backward."""
    n, D = hidden.shape
    V = weight.shape[0]
    dh = torch.empty_like(hidden)
    dw = d_weight if d_weight is not None else torch.empty(
        V, D, dtype=_acc_dtype(hidden.dtype), device=hidden.device)
    ws = workspace if workspace is not None else workspace_for(n, D, V, chunk, hidden.dtype,
                                                               hidden.device)
    st = lce_backward(hidden, weight, targets, loss_mask, lse, n, D, V, chunk, z_coef, grad_out,
                      dh, dw, accumulate, ws)
    if st != OK:
        raise LceError(st, "lce_backward")
    return dh, dw


def forward_backward(hidden, weight, targets, loss_mask=None, chunk=256, z_coef=0.0,
                     grad_out=1.0, d_weight=None, accumulate=False, workspace=None):
    """Allocate lse, d_hidden, d_weight (unless given) and the workspace, call
    lce_forward_backward.  Returns (ForwardResult, d_hidden, d_weight)."""
    n, D = hidden.shape
    V = weight.shape[0]
    acc = _acc_dtype(hidden.dtype)
    lse = torch.empty(n, dtype=acc, device=hidden.device)
    dh = torch.empty_like(hidden)
    dw = d_weight if d_weight is not None else torch.empty(V, D, dtype=acc, device=hidden.device)
    if workspace is None:
        nbytes = lce_forward_backward_workspace_bytes(n, D, V, chunk, hidden.dtype)
        if nbytes < 0:
            raise LceError(int(-nbytes), "lce_forward_backward_workspace_bytes")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=hidden.device)
    st, out = lce_forward_backward(hidden, weight, targets, loss_mask, n, D, V, chunk, z_coef,
                                   grad_out, lse, dh, dw, accumulate, workspace)
    if st != OK:
        raise LceError(st, "lce_forward_backward")
    return ForwardResult(out.as_dict(), lse), dh, dw


def distill(student, teacher, loss_mask=None, objective=0, temperature=1.0, z_coef=0.0,
            grad_out=1.0, workspace=None):
    """Allocate grad_logits and the workspace, call lce_distill_fwd_bwd."""
    n, V = student.shape
    g = torch.empty_like(student)
    nbytes = lce_distill_workspace_bytes(n, V)
    if nbytes < 0:
        raise LceError(int(-nbytes), "lce_distill_workspace_bytes")
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8,
                                                             device=student.device)
    st, out = lce_distill_fwd_bwd(student, teacher, loss_mask, n, V, objective, temperature,
                                  z_coef, grad_out, g, ws)
    if st != OK:
        raise LceError(st, "lce_distill_fwd_bwd")
    return out.as_dict(), g


def ce_logits(logits, targets, loss_mask=None, z_coef=0.0, grad_out=1.0, want_grad=True,
              workspace=None):
    """Label cross-entropy + z-loss from materialized logits [n][V]: allocate
    grad_logits (unless want_grad is False) and the workspace, call
    lce_ce_logits_fwd_bwd.  Returns (loss dict, grad_logits or None)."""
    n, V = logits.shape
    g = torch.empty_like(logits) if want_grad else None
    nbytes = lce_distill_workspace_bytes(n, V)
    if nbytes < 0:
        raise LceError(int(-nbytes), "lce_distill_workspace_bytes")
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8,
                                                             device=logits.device)
    st, out = lce_ce_logits_fwd_bwd(logits, targets, loss_mask, n, V, z_coef, grad_out, g, ws)
    if st != OK:
        raise LceError(st, "lce_ce_logits_fwd_bwd")
    return out.as_dict(), g
