"""CPU fp64 oracle for fused linear cross-entropy (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product package
``lm_head_linear_amd`` never does.  The arithmetic lives in ``lce_oracle.c``
(plain C, fp64, ascending-order sums); this file only marshals numpy arrays.
It shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lce_oracle.c")
_LIB = os.path.join(_HERE, "liblce_oracle.so")

OK = 580


def build(force: bool = True) -> str:
    """Compile lce_oracle.c with gcc (plain fp64, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.orc_status_name.restype = ctypes.c_char_p
        lib.orc_status_name.argtypes = [i32]
        lib.orc_work_fits.argtypes = [i64, i64, i64, i64]
        lib.orc_dims_check.argtypes = [i64, i64, i64]
        lib.orc_chunk_check.argtypes = [i64, i64]
        lib.orc_logit_cells.restype = dbl
        lib.orc_logit_cells.argtypes = [i64, i64]
        lib.orc_peak_cells.argtypes = [i64, i64, i64, vp, vp]
        lib.orc_targets_in_range.argtypes = [vp, i64, i64]
        lib.orc_ce_from_logits.argtypes = [vp, vp, i64, i64, vp, vp]
        lib.orc_fused_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, dbl, i32,
                                          vp, vp, vp]
        lib.orc_backward_dh_rows.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, dbl, dbl,
                                             vp, i64, i32, vp]
        lib.orc_backward_dw_rows.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, dbl, dbl,
                                             vp, i64, i32, i32, vp]
        lib.orc_distill.argtypes = [vp, vp, vp, i64, i64, i32, dbl, dbl, dbl, i32, vp, vp]
        lib.orc_distill_rows.argtypes = [vp, vp, vp, i64, i32, dbl, dbl, dbl, i64, vp, i64,
                                         i32, vp, vp, vp]
        lib.orc_ce_logits.argtypes = [vp, vp, vp, i64, i64, dbl, dbl, i32, vp, vp]
        lib.orc_ce_logits_rows.argtypes = [vp, vp, vp, i64, i64, dbl, dbl, i64, i32, vp, vp, vp]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _mask(m):
    if m is None:
        return None
    return np.ascontiguousarray(m, dtype=np.uint8)


def _p(a):
    return None if a is None else a.ctypes.data


# ---------------------------------------------------------------- contract --

def status_name(code: int) -> str:
    return _load().orc_status_name(int(code)).decode()


def work_fits(n, d, v, ceiling) -> bool:
    return bool(_load().orc_work_fits(n, d, v, ceiling))


def dims_check(n_tok, d_model, vocab) -> int:
    return _load().orc_dims_check(n_tok, d_model, vocab)


def chunk_check(chunk, vocab) -> int:
    return _load().orc_chunk_check(chunk, vocab)


def logit_cells(chunk, vocab) -> float:
    return _load().orc_logit_cells(chunk, vocab)


def peak_cells(n_tok, vocab, chunk) -> dict:
    out = np.zeros(3, dtype=np.float64)
    nch = np.zeros(1, dtype=np.int64)
    st = _load().orc_peak_cells(n_tok, vocab, chunk, out.ctypes.data, nch.ctypes.data)
    return {"chunked_cells": float(out[0]), "materialized_cells": float(out[1]),
            "ratio": float(out[2]), "n_chunks": int(nch[0]), "status": int(st)}


def targets_in_range(targets, n_tok, vocab) -> bool:
    t = _i64(targets)
    assert t.size >= n_tok
    return bool(_load().orc_targets_in_range(t.ctypes.data, n_tok, vocab))


# ---------------------------------------------------------------- compute --

def ce_from_logits(logits, targets):
    """Cross-entropy from materialized logits [n][V] -> (status, mean, per-token)."""
    L = _f64(logits)
    n, V = L.shape
    y = _i64(targets)
    per = np.zeros(n, dtype=np.float64)
    mean = np.zeros(1, dtype=np.float64)
    st = _load().orc_ce_from_logits(L.ctypes.data, y.ctypes.data, n, V, per.ctypes.data,
                                    mean.ctypes.data)
    return st, float(mean[0]), per


def fused_forward(H, W, targets, mask=None, chunk=None, z_coef=0.0, nthreads=None):
    """Chunked fused forward.  Returns dict with status, loss_sum, loss_mean,
    z_sum, z_mean, n_counted, lse[n], loss_tok[n]."""
    H = _f64(H)
    W = _f64(W)
    y = _i64(targets)
    m = _mask(mask)
    n, D = H.shape
    V = W.shape[0]
    assert W.shape[1] == D and y.size == n
    if chunk is None:
        chunk = n
    lse = np.zeros(n, dtype=np.float64)
    lt = np.zeros(n, dtype=np.float64)
    out = np.zeros(5, dtype=np.float64)
    st = _load().orc_fused_forward(H.ctypes.data, W.ctypes.data, y.ctypes.data, _p(m), n, D,
                                   V, int(chunk), float(z_coef),
                                   nthreads or default_threads(), lse.ctypes.data,
                                   lt.ctypes.data, out.ctypes.data)
    return {"status": int(st), "loss_sum": float(out[0]), "loss_mean": float(out[1]),
            "z_sum": float(out[2]), "z_mean": float(out[3]), "n_counted": int(out[4]),
            "lse": lse, "loss_tok": lt}


def backward_dh_rows(H, W, targets, lse, rows, mask=None, z_coef=0.0, grad_out=1.0,
                     nthreads=None):
    H = _f64(H)
    W = _f64(W)
    y = _i64(targets)
    m = _mask(mask)
    lse = _f64(lse)
    rows = _i64(rows)
    n, D = H.shape
    V = W.shape[0]
    out = np.zeros((rows.size, D), dtype=np.float64)
    st = _load().orc_backward_dh_rows(H.ctypes.data, W.ctypes.data, y.ctypes.data, _p(m),
                                      lse.ctypes.data, n, D, V, float(z_coef),
                                      float(grad_out), rows.ctypes.data, rows.size,
                                      nthreads or default_threads(), out.ctypes.data)
    assert st == OK, st
    return out


def backward_dw_rows(H, W, targets, lse, rows, mask=None, z_coef=0.0, grad_out=1.0,
                     dw_in=None, nthreads=None):
    H = _f64(H)
    W = _f64(W)
    y = _i64(targets)
    m = _mask(mask)
    lse = _f64(lse)
    rows = _i64(rows)
    n, D = H.shape
    V = W.shape[0]
    if dw_in is None:
        out = np.zeros((rows.size, D), dtype=np.float64)
        acc = 0
    else:
        out = np.array(dw_in, dtype=np.float64, copy=True).reshape(rows.size, D)
        acc = 1
    st = _load().orc_backward_dw_rows(H.ctypes.data, W.ctypes.data, y.ctypes.data, _p(m),
                                      lse.ctypes.data, n, D, V, float(z_coef),
                                      float(grad_out), rows.ctypes.data, rows.size, acc,
                                      nthreads or default_threads(), out.ctypes.data)
    assert st == OK, st
    return out


def backward(H, W, targets, lse, mask=None, z_coef=0.0, grad_out=1.0, dw_in=None,
             nthreads=None):
    """Full d_hidden [n][D] and d_weight [V][D]."""
    n = np.asarray(H).shape[0]
    V = np.asarray(W).shape[0]
    dH = backward_dh_rows(H, W, targets, lse, np.arange(n), mask, z_coef, grad_out, nthreads)
    dW = backward_dw_rows(H, W, targets, lse, np.arange(V), mask, z_coef, grad_out, dw_in,
                          nthreads)
    return dH, dW


def distill(S, U, mask=None, objective=0, temperature=1.0, z_coef=0.0, grad_out=1.0,
            want_grad=True, nthreads=None):
    """Distillation loss and gradient over full [n][V] student/teacher logits."""
    S = _f64(S)
    U = _f64(U)
    m = _mask(mask)
    n, V = S.shape
    assert U.shape == S.shape
    grad = np.zeros((n, V), dtype=np.float64) if want_grad else None
    out = np.zeros(5, dtype=np.float64)
    st = _load().orc_distill(S.ctypes.data, U.ctypes.data, _p(m), n, V, int(objective),
                             float(temperature), float(z_coef), float(grad_out),
                             nthreads or default_threads(), _p(grad), out.ctypes.data)
    return {"status": int(st), "loss": float(out[0]), "z_loss": float(out[1]),
            "n_counted": int(out[2]), "loss_sum": float(out[3]), "z_sum": float(out[4]),
            "grad": grad}


def distill_rows(S_rows, U_rows, n_counted, row_mask=None, objective=0, temperature=1.0,
                 z_coef=0.0, grad_out=1.0, nthreads=None):
    """Distillation on selected rows of a larger batch.

    S_rows/U_rows hold only the selected rows [k][V]; row_mask their mask
    flags; n_counted is the divisor C of the whole batch.
    Returns (grad_rows [k][V], row_loss [k], row_lse [k])."""
    S = _f64(S_rows)
    U = _f64(U_rows)
    m = _mask(row_mask)
    k, V = S.shape
    rows = np.arange(k, dtype=np.int64)
    g = np.zeros((k, V), dtype=np.float64)
    rl = np.zeros(k, dtype=np.float64)
    rz = np.zeros(k, dtype=np.float64)
    st = _load().orc_distill_rows(S.ctypes.data, U.ctypes.data, _p(m), V, int(objective),
                                  float(temperature), float(z_coef), float(grad_out),
                                  int(n_counted), rows.ctypes.data, k,
                                  nthreads or default_threads(), g.ctypes.data,
                                  rl.ctypes.data, rz.ctypes.data)
    assert st == OK, st
    return g, rl, rz


def ce_logits(Z, targets, mask=None, z_coef=0.0, grad_out=1.0, want_grad=True, nthreads=None):
    """Label cross-entropy + z-loss from materialized logits [n][V], forward
    and backward (the lossk reference function with the mask and z term)."""
    Z = _f64(Z)
    y = _i64(targets)
    m = _mask(mask)
    n, V = Z.shape
    grad = np.zeros((n, V), dtype=np.float64) if want_grad else None
    out = np.zeros(5, dtype=np.float64)
    st = _load().orc_ce_logits(Z.ctypes.data, y.ctypes.data, _p(m), n, V, float(z_coef),
                               float(grad_out), nthreads or default_threads(), _p(grad),
                               out.ctypes.data)
    return {"status": int(st), "loss": float(out[0]), "z_loss": float(out[1]),
            "n_counted": int(out[2]), "loss_sum": float(out[3]), "z_sum": float(out[4]),
            "grad": grad}


def ce_logits_rows(Z_rows, targets_rows, n_counted, row_mask=None, z_coef=0.0, grad_out=1.0,
                   nthreads=None):
    """ce_logits on selected rows of a larger batch (n_counted = its divisor C).
    Returns (grad_rows [k][V], row_loss [k], row_lse [k])."""
    Z = _f64(Z_rows)
    y = _i64(targets_rows)
    m = _mask(row_mask)
    k, V = Z.shape
    g = np.zeros((k, V), dtype=np.float64)
    rl = np.zeros(k, dtype=np.float64)
    rz = np.zeros(k, dtype=np.float64)
    st = _load().orc_ce_logits_rows(Z.ctypes.data, y.ctypes.data, _p(m), k, V, float(z_coef),
                                    float(grad_out), int(n_counted),
                                    nthreads or default_threads(), g.ctypes.data,
                                    rl.ctypes.data, rz.ctypes.data)
    assert st == OK, st
    return g, rl, rz
