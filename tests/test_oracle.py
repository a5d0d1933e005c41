"""Pins for the CPU fp64 oracle (no GPU).

Every oracle function is checked here against something other than itself:
values printed on the pages (tests/golden/), closed forms, exact integer
arithmetic, torch CPU fp64 library routines, finite differences and
identities of the mathematics.  Each check is chosen so that a dropped term,
a wrong sign or index or a transposed operand in the oracle fails it.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ------------------------------------------------------------ contract pins --

def test_printed_budget_values():
    for row in _read_golden("p1_budgets.txt"):
        lhs, rhs = row.split("->")
        kind, *args = lhs.split()
        args = [int(a) for a in args]
        exp = rhs.split()
        if kind == "peak":
            r = oracle.peak_cells(*args)
            assert r["chunked_cells"] == float(exp[0])
            assert r["materialized_cells"] == float(exp[1])
            assert r["ratio"] == float(exp[2])
            assert r["n_chunks"] == int(exp[3])
            assert r["status"] == int(exp[4])
        elif kind == "dims":
            assert oracle.dims_check(*args) == int(exp[0])
        elif kind == "chunk":
            assert oracle.chunk_check(*args) == int(exp[0])
        else:
            raise AssertionError(kind)


def test_chunk_check_exact_boundary():
    # 2^27 / 151936 = 883.4: 883 rows fit, 884 do not; 1024 (a swept chunk) does not.
    assert oracle.chunk_check(883, 151936) == 580
    assert oracle.chunk_check(884, 151936) == 587
    assert oracle.chunk_check(1024, 151936) == 587
    assert oracle.chunk_check(512, 128256) == 580
    # equality with the ceiling passes
    assert oracle.chunk_check(2 ** 10, 2 ** 17) == 580
    assert oracle.chunk_check(2 ** 10 + 1, 2 ** 17) == 587
    assert oracle.chunk_check(0, 10) == 581
    assert oracle.chunk_check(10, 0) == 581
    assert oracle.chunk_check(-5, 10) == 581


def test_chunk_and_work_against_exact_integers():
    # Python integers never overflow: compare the divide-down checks with the
    # plain products over a seeded sweep that includes huge values.
    rng = np.random.default_rng(7)
    cases = [(int(a), int(b)) for a, b in rng.integers(1, 2 ** 31, size=(300, 2))]
    cases += [(int(a), int(b)) for a, b in rng.integers(1, 5000, size=(300, 2))]
    cases += [(2 ** 62, 3), (3, 2 ** 62), (2 ** 27, 1), (2 ** 27 + 1, 1), (1, 2 ** 27)]
    for c, v in cases:
        want = 587 if c * v > 2 ** 27 else 580
        assert oracle.chunk_check(c, v) == want, (c, v)
    big = [(2 ** 24, 2 ** 16, 2 ** 6), (2 ** 24, 2 ** 16, 2 ** 6 + 1), (2 ** 40, 2 ** 40, 2 ** 40),
           (2 ** 46, 1, 1), (2 ** 46 + 1, 1, 1), (3, 5, 7)]
    big += [tuple(int(x) for x in r) for r in rng.integers(1, 2 ** 20, size=(300, 3))]
    for n, d, v in big:
        assert oracle.work_fits(n, d, v, 2 ** 46) == (n * d * v <= 2 ** 46), (n, d, v)


def test_dims_check_statuses():
    assert oracle.dims_check(0, 1, 1) == 581
    assert oracle.dims_check(1, 0, 1) == 581
    assert oracle.dims_check(1, 1, -1) == 581
    assert oracle.dims_check(2 ** 24, 1, 1) == 580
    assert oracle.dims_check(2 ** 24 + 1, 1, 1) == 583
    assert oracle.dims_check(1, 2 ** 16 + 1, 1) == 583
    assert oracle.dims_check(1, 1, 2 ** 24 + 1) == 583
    # 2^24 * 2^16 * 2^6 = 2^46 exactly: fits; one more vocab row does not
    assert oracle.dims_check(2 ** 24, 2 ** 16, 2 ** 6) == 580
    assert oracle.dims_check(2 ** 24, 2 ** 16, 2 ** 6 + 1) == 584
    assert oracle.dims_check(8192, 4096, 128256) == 580


def test_peak_cells_edges():
    r = oracle.peak_cells(0, 10, 4)
    assert r == {"chunked_cells": -1.0, "materialized_cells": -1.0, "ratio": -1.0,
                 "n_chunks": 0, "status": 581}
    r = oracle.peak_cells(10, 7, 3)          # ragged last chunk
    assert r["n_chunks"] == 4 and r["chunked_cells"] == 21.0 and r["ratio"] == 70.0 / 21.0
    r = oracle.peak_cells(10, 7, 50)         # chunk larger than the batch holds the batch
    assert r["chunked_cells"] == 70.0 and r["ratio"] == 1.0 and r["n_chunks"] == 1
    r = oracle.peak_cells(2048, 151936, 2048)
    assert r["status"] == 587 and r["materialized_cells"] == 311164928.0
    assert oracle.logit_cells(0, 5) == -1.0 and oracle.logit_cells(256, 151936) == 38895616.0


def test_status_names():
    names = {580: "ok", 581: "empty_dimension", 582: "length_mismatch",
             583: "dimension_too_large", 584: "work_budget_exceeded",
             585: "non_finite_scalar", 586: "target_id_out_of_range",
             587: "chunk_exceeds_logit_budget", 588: "unknown_objective"}
    for k, v in names.items():
        assert oracle.status_name(k) == v
    assert oracle.status_name(579) == "unknown_status"
    assert oracle.status_name(600) == "unknown_status"


def test_targets_guard():
    assert oracle.targets_in_range([0, 5, 9], 3, 10)
    assert not oracle.targets_in_range([0, 10, 9], 3, 10)
    assert not oracle.targets_in_range([0, -1, 9], 3, 10)   # negative is refused, not a mask
    assert oracle.targets_in_range([0, 1, -1], 2, 10)        # only the first n_tok are read


# --------------------------------------------------- cross-entropy from logits --

def test_uniform_logits_golden_bit_exact():
    g = dict(r.split(None, 1) for r in _read_golden("p1_uniform_logits.txt"))
    n, V = int(g["n_tok"]), int(g["vocab"])
    logits = np.full((n, V), float(g["logit"]))
    y = [int(x) for x in g["targets"].split()]
    st, mean, per = oracle.ce_from_logits(logits, y)
    assert st == 580
    assert mean == float(g["mean_loss"])          # bit-exact, as printed
    assert mean == math.log(9)


@pytest.mark.parametrize("V", [1, 2, 1000, 151936])
def test_all_equal_logits_give_log_vocab(V):
    st, mean, per = oracle.ce_from_logits(np.zeros((3, V)), [0, V // 2, V - 1])
    assert st == 580 and np.all(per == math.log(V)) and mean == math.log(V)


def test_ce_from_logits_matches_torch():
    rng = np.random.default_rng(11)
    L = rng.standard_normal((17, 203)) * 3.0
    y = rng.integers(0, 203, 17)
    st, mean, per = oracle.ce_from_logits(L, y)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(L), torch.from_numpy(y),
                                            reduction="none").numpy()
    assert st == 580
    np.testing.assert_allclose(per, ref, rtol=1e-13, atol=0)
    assert abs(mean - ref.mean()) <= 1e-13 * abs(ref.mean())


def test_ce_from_logits_refusals():
    assert oracle.ce_from_logits(np.zeros((2, 4)), [0, 4])[0] == 586
    assert oracle.ce_from_logits(np.zeros((2, 4)), [-1, 0])[0] == 586


# -------------------------------------------------------- fused forward --

def _tiny(n=6, D=5, V=11, seed=0, mask_frac=0.0):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((n, D))
    W = rng.standard_normal((V, D)) * 0.5
    y = rng.integers(0, V, n)
    m = syn.exact_mask(rng, n, mask_frac)
    return H, W, y, m


def _py_logits(H, W):
    """Logits by pure-Python loops, ascending d, product then sum."""
    n, D = H.shape
    V = W.shape[0]
    out = np.zeros((n, V))
    for t in range(n):
        for v in range(V):
            acc = 0.0
            for d in range(D):
                acc = acc + float(W[v, d]) * float(H[t, d])
            out[t, v] = acc
    return out


def test_fused_equals_materialized_bit_exact():
    H, W, y, _ = _tiny()
    st, mean, per = oracle.ce_from_logits(_py_logits(H, W), y)
    for chunk in (1, 2, 3, 6, 100):
        r = oracle.fused_forward(H, W, y, chunk=chunk)
        assert r["status"] == 580
        assert np.array_equal(r["loss_tok"], per)
        assert r["loss_mean"] == mean


def test_fused_forward_matches_torch():
    H, W, y, m = _tiny(n=40, D=24, V=301, seed=3, mask_frac=0.25)
    r = oracle.fused_forward(H, W, y, mask=m, chunk=7, z_coef=1e-2)
    Ht, Wt = torch.from_numpy(H), torch.from_numpy(W)
    logits = Ht @ Wt.T
    lse = torch.logsumexp(logits, dim=1).numpy()
    per = torch.nn.functional.cross_entropy(logits, torch.from_numpy(y), reduction="none").numpy()
    keep = m.astype(bool)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-13)
    assert r["n_counted"] == keep.sum() == 30
    assert abs(r["loss_mean"] - per[keep].mean()) <= 1e-13 * abs(per[keep].mean())
    assert abs(r["z_mean"] - (lse[keep] ** 2).mean()) <= 1e-13 * (lse[keep] ** 2).mean()


def test_chunk_invariance_every_chunk_tiny_workload():
    w = syn.TINY_F64
    x = syn.ce_inputs(w)
    H, W = x.hidden64(), x.weight64()
    base = oracle.fused_forward(H, W, x.targets, chunk=1, nthreads=4)
    assert base["status"] == 580
    for chunk in range(2, w.n_tok + 1):
        r = oracle.fused_forward(H, W, x.targets, chunk=chunk, nthreads=4)
        assert r["loss_mean"] == base["loss_mean"], chunk      # max_abs_delta == 0.0
        assert np.array_equal(r["lse"], base["lse"])


def test_thread_count_does_not_change_bits():
    H, W, y, m = _tiny(n=37, D=19, V=257, seed=5, mask_frac=0.2)
    a = oracle.fused_forward(H, W, y, mask=m, chunk=5, z_coef=1e-3, nthreads=1)
    b = oracle.fused_forward(H, W, y, mask=m, chunk=5, z_coef=1e-3, nthreads=7)
    assert a["loss_mean"] == b["loss_mean"] and np.array_equal(a["lse"], b["lse"])
    g1 = oracle.backward(H, W, y, a["lse"], mask=m, z_coef=1e-3, nthreads=1)
    g7 = oracle.backward(H, W, y, a["lse"], mask=m, z_coef=1e-3, nthreads=7)
    assert np.array_equal(g1[0], g7[0]) and np.array_equal(g1[1], g7[1])


@pytest.mark.parametrize("V", [1000, 151936])
def test_zero_weight_gives_log_vocab_and_z(V):
    n, D = 5, 3
    H = np.random.default_rng(0).standard_normal((n, D))
    W = np.zeros((V, D))
    y = np.arange(n) * (V // n)
    r = oracle.fused_forward(H, W, y, chunk=2, z_coef=1e-4)
    assert np.all(r["loss_tok"] == math.log(V)) and r["loss_mean"] == math.log(V)
    assert np.all(r["lse"] == math.log(V))
    z_expect = {1000: 47.71708299430558, 151936: 142.35388322790408}[V]
    assert r["z_mean"] == pytest.approx(z_expect, rel=1e-15)
    assert r["z_mean"] == pytest.approx(math.log(V) ** 2, rel=1e-15)


def test_mask_equals_compaction_and_all_true():
    H, W, y, m = _tiny(n=23, D=9, V=131, seed=8, mask_frac=0.3)
    r = oracle.fused_forward(H, W, y, mask=m, chunk=4, z_coef=0.01)
    keep = m.astype(bool)
    c = oracle.fused_forward(H[keep], W, y[keep], chunk=4, z_coef=0.01)
    assert r["loss_mean"] == c["loss_mean"] and r["z_mean"] == c["z_mean"]
    assert r["n_counted"] == keep.sum()
    a = oracle.fused_forward(H, W, y, mask=np.ones(23, np.uint8), chunk=4)
    b = oracle.fused_forward(H, W, y, chunk=4)
    assert a["loss_mean"] == b["loss_mean"]
    z = oracle.fused_forward(H, W, y, mask=np.zeros(23, np.uint8), chunk=4)
    assert z["status"] == 580 and z["loss_mean"] == 0.0 and z["z_mean"] == 0.0
    assert z["n_counted"] == 0


def test_fused_forward_refusals():
    H, W, y, _ = _tiny()
    assert oracle.fused_forward(H, W, y, chunk=0)["status"] == 581
    assert oracle.fused_forward(H, W, y, z_coef=float("nan"))["status"] == 585
    assert oracle.fused_forward(H, W, y, z_coef=float("inf"))["status"] == 585
    bad = y.copy()
    bad[2] = W.shape[0]
    assert oracle.fused_forward(H, W, bad)["status"] == 586
    bad[2] = -1
    assert oracle.fused_forward(H, W, bad)["status"] == 586
    Wbig = np.zeros((140000, 1))
    assert oracle.fused_forward(np.zeros((2, 1)), Wbig, [0, 1], chunk=1000)["status"] == 587


# -------------------------------------------------------------- backward --

def _objective(H, W, y, m, z_coef, grad_out):
    r = oracle.fused_forward(H, W, y, mask=m, chunk=3, z_coef=z_coef, nthreads=1)
    return grad_out * (r["loss_mean"] + z_coef * r["z_mean"])


@pytest.mark.parametrize("z_coef,mask_frac,grad_out", [(0.0, 0.0, 1.0), (0.05, 0.0, 1.0),
                                                        (0.05, 0.25, 2.5)])
def test_backward_finite_differences(z_coef, mask_frac, grad_out):
    H, W, y, m = _tiny(n=4, D=8, V=16, seed=21, mask_frac=mask_frac)
    r = oracle.fused_forward(H, W, y, mask=m, chunk=3, z_coef=z_coef)
    dH, dW = oracle.backward(H, W, y, r["lse"], mask=m, z_coef=z_coef, grad_out=grad_out)
    h = 1e-5
    for X, G in ((H, dH), (W, dW)):
        fd = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _objective(H, W, y, m, z_coef, grad_out)
            X[idx] = old - h
            fm = _objective(H, W, y, m, z_coef, grad_out)
            X[idx] = old
            fd[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(fd - G)) <= 1e-8


def test_backward_matches_torch_autograd():
    H, W, y, m = _tiny(n=30, D=12, V=97, seed=4, mask_frac=0.2)
    z_coef, grad_out = 0.03, 1.7
    r = oracle.fused_forward(H, W, y, mask=m, chunk=8, z_coef=z_coef)
    dH, dW = oracle.backward(H, W, y, r["lse"], mask=m, z_coef=z_coef, grad_out=grad_out)
    Ht = torch.from_numpy(H.copy()).requires_grad_(True)
    Wt = torch.from_numpy(W.copy()).requires_grad_(True)
    logits = Ht @ Wt.T
    keep = torch.from_numpy(m.astype(bool))
    ce = torch.nn.functional.cross_entropy(logits, torch.from_numpy(y), reduction="none")
    lse = torch.logsumexp(logits, dim=1)
    C = keep.sum()
    obj = grad_out * ((ce * keep).sum() / C + z_coef * ((lse ** 2) * keep).sum() / C)
    obj.backward()
    assert np.max(np.abs(dH - Ht.grad.numpy())) <= 1e-13 * np.max(np.abs(dH))
    assert np.max(np.abs(dW - Wt.grad.numpy())) <= 1e-13 * np.max(np.abs(dW))
    assert np.all(dH[~m.astype(bool)] == 0.0)          # masked rows exactly zero


def test_dweight_cancels_over_vocab():
    x = syn.ce_inputs(syn.TINY_F64)
    H, W = x.hidden64(), x.weight64()
    r = oracle.fused_forward(H, W, x.targets, chunk=16)
    _, dW = oracle.backward(H, W, x.targets, r["lse"])
    assert np.max(np.abs(dW.sum(axis=0))) <= 1e-9
    # with z-loss the column sums equal sum_t 2*g_z*lse_t*H[t]
    z = 1e-2
    r = oracle.fused_forward(H, W, x.targets, chunk=16, z_coef=z)
    _, dWz = oracle.backward(H, W, x.targets, r["lse"], z_coef=z)
    want = (2 * z / H.shape[0]) * (r["lse"][:, None] * H).sum(axis=0)
    assert np.max(np.abs(dWz.sum(axis=0) - want)) <= 1e-9


def test_backward_linear_in_grad_out_and_accumulates():
    H, W, y, m = _tiny(n=9, D=6, V=29, seed=9, mask_frac=0.2)
    r = oracle.fused_forward(H, W, y, mask=m, chunk=4, z_coef=0.1)
    a = oracle.backward(H, W, y, r["lse"], mask=m, z_coef=0.1, grad_out=1.0)
    b = oracle.backward(H, W, y, r["lse"], mask=m, z_coef=0.1, grad_out=4.0)
    np.testing.assert_allclose(b[0], 4 * a[0], rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(b[1], 4 * a[1], rtol=1e-14, atol=1e-300)
    dw_in = np.random.default_rng(1).standard_normal(W.shape)
    c = oracle.backward(H, W, y, r["lse"], mask=m, z_coef=0.1, grad_out=1.0, dw_in=dw_in)
    assert np.array_equal(c[1], dw_in + a[1])


def test_backward_all_masked_is_zero():
    H, W, y, _ = _tiny()
    m = np.zeros(H.shape[0], np.uint8)
    r = oracle.fused_forward(H, W, y, mask=m)
    dH, dW = oracle.backward(H, W, y, r["lse"], mask=m)
    assert not dH.any() and not dW.any()


# ---------------------------------------------------------- distillation --

def _dis_inputs(n=7, V=53, seed=2, mask_frac=0.0):
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((n, V)) * 4.0
    U = S + rng.standard_normal((n, V))
    m = syn.exact_mask(rng, n, mask_frac)
    return S, U, m


@pytest.mark.parametrize("obj", [1, 2])
def test_kl_zero_when_student_equals_teacher(obj):
    S, _, _ = _dis_inputs()
    r = oracle.distill(S, S, objective=obj, temperature=2.0)
    assert r["status"] == 580 and r["loss"] == 0.0 and not r["grad"].any()


def test_ce_minus_forward_kl_is_teacher_entropy():
    S, U, m = _dis_inputs(mask_frac=0.3)
    T = 1.5
    ce = oracle.distill(S, U, mask=m, objective=0, temperature=T)
    fkl = oracle.distill(S, U, mask=m, objective=1, temperature=T)
    y = torch.from_numpy(U / T)
    lq = torch.log_softmax(y, dim=1)
    Hq = -(lq.exp() * lq).sum(dim=1).numpy()
    keep = m.astype(bool)
    assert abs((ce["loss"] - fkl["loss"]) - Hq[keep].mean()) <= 1e-12
    assert np.array_equal(ce["grad"], fkl["grad"])      # same gradient p - q, bit for bit


@pytest.mark.parametrize("obj", [0, 1, 2])
def test_distill_matches_torch(obj):
    S, U, m = _dis_inputs(n=11, V=67, seed=6, mask_frac=0.2)
    T, z, go = 2.0, 0.05, 1.3
    r = oracle.distill(S, U, mask=m, objective=obj, temperature=T, z_coef=z, grad_out=go)
    St = torch.from_numpy(S.copy()).requires_grad_(True)
    x = St / T
    y = torch.from_numpy(U) / T
    ls = torch.log_softmax(x, dim=1)
    lq = torch.log_softmax(y, dim=1)
    if obj == 0:
        Lt = -(lq.exp() * ls).sum(1)
    elif obj == 1:
        Lt = torch.nn.functional.kl_div(ls, lq, reduction="none", log_target=True).sum(1)
    else:
        Lt = torch.nn.functional.kl_div(lq, ls, reduction="none", log_target=True).sum(1)
    keep = torch.from_numpy(m.astype(bool))
    C = keep.sum()
    lse = torch.logsumexp(x, dim=1)
    loss = (Lt * keep).sum() / C
    zl = ((lse ** 2) * keep).sum() / C
    (go * (loss + z * zl)).backward()
    assert abs(r["loss"] - loss.item()) <= 1e-12 * max(1.0, abs(loss.item()))
    assert abs(r["z_loss"] - zl.item()) <= 1e-12 * zl.item()
    g = St.grad.numpy()
    assert np.max(np.abs(r["grad"] - g)) <= 1e-12 * np.max(np.abs(g))


@pytest.mark.parametrize("obj", [0, 1, 2])
def test_distill_finite_differences(obj):
    S, U, m = _dis_inputs(n=3, V=9, seed=12, mask_frac=0.34)
    T, z, go = 1.7, 0.1, 0.9
    r = oracle.distill(S, U, mask=m, objective=obj, temperature=T, z_coef=z, grad_out=go)
    h = 1e-5

    def f():
        q = oracle.distill(S, U, mask=m, objective=obj, temperature=T, z_coef=z,
                           grad_out=go, want_grad=False)
        return go * (q["loss"] + z * q["z_loss"])

    fd = np.zeros_like(S)
    for idx in np.ndindex(*S.shape):
        old = S[idx]
        S[idx] = old + h
        fp = f()
        S[idx] = old - h
        fm = f()
        S[idx] = old
        fd[idx] = (fp - fm) / (2 * h)
    assert np.max(np.abs(fd - r["grad"])) <= 1e-8


@pytest.mark.parametrize("obj", [0, 1, 2])
def test_temperature_scaling_identity(obj):
    S, U, m = _dis_inputs(seed=13, mask_frac=0.2)
    T = 2.0   # a power of two, so S/T is exact and the identity holds bit for bit
    a = oracle.distill(S, U, mask=m, objective=obj, temperature=T, z_coef=0.01)
    b = oracle.distill(S / T, U / T, mask=m, objective=obj, temperature=1.0, z_coef=0.01)
    assert a["loss"] == b["loss"] and a["z_loss"] == b["z_loss"]
    assert np.array_equal(a["grad"], b["grad"] / T)


def test_one_hot_teacher_limit_is_label_ce():
    rng = np.random.default_rng(14)
    n, V = 6, 40
    S = rng.standard_normal((n, V))
    y = rng.integers(0, V, n)
    U = np.zeros((n, V))
    U[np.arange(n), y] = 60.0        # teacher mass off the label ~ V*e^-60
    r = oracle.distill(S, U, objective=0, temperature=1.0)
    st, mean, _ = oracle.ce_from_logits(S, y)
    assert abs(r["loss"] - mean) <= 1e-20 * V + 1e-14


def test_distill_z_term_is_additive():
    S, U, m = _dis_inputs(seed=15, mask_frac=0.2)
    for obj in (0, 1, 2):
        off = oracle.distill(S, U, mask=m, objective=obj, temperature=1.5, z_coef=0.0)
        on = oracle.distill(S, U, mask=m, objective=obj, temperature=1.5, z_coef=0.2)
        zonly = on["grad"] - off["grad"]
        # the z-only gradient: (grad_out/C) * 2 z lse(x) p / T
        x = torch.from_numpy(S / 1.5)
        p = torch.softmax(x, 1).numpy()
        lse = torch.logsumexp(x, 1).numpy()
        keep = m.astype(bool)
        want = (1.0 / keep.sum()) * 2 * 0.2 * lse[:, None] * p / 1.5 * keep[:, None]
        assert np.max(np.abs(zonly - want)) <= 1e-14
        assert on["loss"] == off["loss"]


def test_distill_refusals_and_rows():
    S, U, m = _dis_inputs(mask_frac=0.3)
    assert oracle.distill(S, U, objective=3)["status"] == 588
    assert oracle.distill(S, U, temperature=0.0)["status"] == 585
    assert oracle.distill(S, U, temperature=-1.0)["status"] == 585
    assert oracle.distill(S, U, temperature=float("nan"))["status"] == 585
    assert oracle.distill(S, U, z_coef=float("inf"))["status"] == 585
    full = oracle.distill(S, U, mask=m, objective=2, temperature=2.0, z_coef=0.1)
    rows = np.array([0, 3, 6])
    g, rl, rz = oracle.distill_rows(S[rows], U[rows], full["n_counted"], row_mask=m[rows],
                                    objective=2, temperature=2.0, z_coef=0.1)
    assert np.array_equal(g, full["grad"][rows])


# ------------------------------------ label cross-entropy + z from logits --

def test_ce_logits_uniform_golden_and_closed_form():
    """The lossk worked example (9 equal logits -> log 9, bit-exact) and the
    closed form of every term for equal logits c: lse = c + log V, z = lse^2,
    grad = (g/C)((1 + 2 z_coef lse)/V - onehot)."""
    g = dict(r.split(None, 1) for r in _read_golden("p1_uniform_logits.txt"))
    n, V = int(g["n_tok"]), int(g["vocab"])
    y = [int(x) for x in g["targets"].split()]
    r = oracle.ce_logits(np.full((n, V), float(g["logit"])), y)
    assert r["status"] == 580 and r["loss"] == float(g["mean_loss"])
    c, V, zc, go = 1.5, 7, 0.25, 1.75
    y = np.array([0, 3, 6, 2])
    m = np.array([1, 1, 0, 1], dtype=np.uint8)
    r = oracle.ce_logits(np.full((4, V), c), y, mask=m, z_coef=zc, grad_out=go)
    lse = c + math.log(V)
    assert r["n_counted"] == 3
    assert abs(r["loss"] - math.log(V)) <= 1e-15
    assert abs(r["z_loss"] - lse * lse) <= 1e-14
    want = np.full((4, V), (go / 3) * (1 + 2 * zc * lse) / V)
    want[np.arange(4), y] -= go / 3
    want[2] = 0.0
    assert np.max(np.abs(r["grad"] - want)) <= 1e-15


def test_ce_logits_loss_matches_ce_from_logits():
    rng = np.random.default_rng(21)
    Z = rng.standard_normal((13, 301)) * 4.0
    y = rng.integers(0, 301, 13)
    r = oracle.ce_logits(Z, y, want_grad=False)
    st, mean, per = oracle.ce_from_logits(Z, y)
    assert r["status"] == st == 580 and r["loss"] == mean


@pytest.mark.parametrize("z_coef,mask_frac", [(0.0, 0.0), (0.3, 0.34)])
def test_ce_logits_finite_differences(z_coef, mask_frac):
    rng = np.random.default_rng(22)
    n, V, go = 3, 8, 1.3
    Z = rng.standard_normal((n, V)) * 2.0
    y = rng.integers(0, V, n)
    m = (rng.random(n) >= mask_frac).astype(np.uint8)
    m[0] = 1
    r = oracle.ce_logits(Z, y, mask=m, z_coef=z_coef, grad_out=go)
    h = 1e-5

    def f():
        q = oracle.ce_logits(Z, y, mask=m, z_coef=z_coef, grad_out=go, want_grad=False)
        return go * (q["loss"] + z_coef * q["z_loss"])

    fd = np.zeros_like(Z)
    for idx in np.ndindex(*Z.shape):
        old = Z[idx]
        Z[idx] = old + h
        fp = f()
        Z[idx] = old - h
        fm = f()
        Z[idx] = old
        fd[idx] = (fp - fm) / (2 * h)
    assert np.max(np.abs(fd - r["grad"])) <= 1e-8


def test_ce_logits_matches_torch_autograd():
    rng = np.random.default_rng(23)
    n, V, zc, go = 9, 57, 1e-2, 0.7
    Z = rng.standard_normal((n, V)) * 3.0
    y = rng.integers(0, V, n)
    m = (rng.random(n) > 0.2).astype(np.uint8)
    r = oracle.ce_logits(Z, y, mask=m, z_coef=zc, grad_out=go)
    Zt = torch.from_numpy(Z.copy()).requires_grad_(True)
    keep = torch.from_numpy(m.astype(bool))
    lse = torch.logsumexp(Zt, 1)
    ce = lse - Zt[torch.arange(n), torch.from_numpy(y)]
    C = int(keep.sum())
    loss = ce[keep].sum() / C
    zl = (lse[keep] ** 2).sum() / C
    (go * (loss + zc * zl)).backward()
    assert abs(r["loss"] - float(loss)) <= 1e-14 * abs(float(loss))
    assert abs(r["z_loss"] - float(zl)) <= 1e-14 * abs(float(zl))
    g = Zt.grad.numpy()
    assert np.max(np.abs(r["grad"] - g)) <= 1e-14 * np.max(np.abs(g))


def test_ce_logits_equals_distill_with_one_hot_teacher():
    """A teacher with all its mass on the label (exp(-800) underflows to 0)
    makes the distillation cross-entropy the label loss, term for term."""
    rng = np.random.default_rng(24)
    n, V = 7, 33
    Z = rng.standard_normal((n, V)) * 2.0
    y = rng.integers(0, V, n)
    m = (rng.random(n) > 0.3).astype(np.uint8)
    U = np.zeros((n, V))
    U[np.arange(n), y] = 800.0
    d = oracle.distill(Z, U, mask=m, objective=0, temperature=1.0, z_coef=0.2, grad_out=1.1)
    r = oracle.ce_logits(Z, y, mask=m, z_coef=0.2, grad_out=1.1)
    assert abs(r["loss"] - d["loss"]) <= 1e-14 and r["z_loss"] == d["z_loss"]
    assert np.max(np.abs(r["grad"] - d["grad"])) <= 1e-16


def test_ce_logits_refusals_and_rows():
    rng = np.random.default_rng(25)
    Z = rng.standard_normal((8, 16))
    y = rng.integers(0, 16, 8)
    m = (rng.random(8) > 0.3).astype(np.uint8)
    assert oracle.ce_logits(Z, np.where(np.arange(8) == 3, 16, y))["status"] == 586
    assert oracle.ce_logits(Z, np.where(np.arange(8) == 5, -1, y))["status"] == 586
    assert oracle.ce_logits(Z, y, z_coef=float("nan"))["status"] == 585
    assert oracle.ce_logits(Z, y, grad_out=float("inf"))["status"] == 585
    full = oracle.ce_logits(Z, y, mask=m, z_coef=0.1, grad_out=2.0)
    rows = np.array([0, 2, 7])
    g, rl, rz = oracle.ce_logits_rows(Z[rows], y[rows], full["n_counted"], row_mask=m[rows],
                                      z_coef=0.1, grad_out=2.0)
    assert np.array_equal(g, full["grad"][rows])


def test_large_golden_file_matches_the_oracle():
    """The stored lse of the 8192 x 4096 x 128256 workload (written by
    tests/golden/make_large_bf16_lse.py) is the oracle's: three tokens
    recomputed here agree to the last bit (per-token dots and the vocabulary
    reduction do not depend on which tokens run together)."""
    import os
    from tests import synthetic as syn
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "large_head_bf16_8192x4096x128256_lse.txt")
    lines = [l for l in open(path) if not l.startswith("#")]
    k = lines.index("lse\n")
    lse = np.array([float(v) for v in lines[k + 1:]])
    assert lse.shape == (8192,)
    w = syn.LARGE_BF16
    x = syn.ce_inputs(w)
    toks = np.array([0, 4095, 8191])
    H = x.hidden[toks].double().numpy()
    r = oracle.fused_forward(H, x.weight64(), x.targets[toks], chunk=3, z_coef=w.z_coef)
    assert r["status"] == 580
    assert np.array_equal(r["lse"], lse[toks])
