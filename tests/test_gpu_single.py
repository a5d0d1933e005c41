"""GPU parity of lce_forward_backward (forward and backward in one call)
against the CPU fp64 oracle, through the C ABI, and against the two-call path
(lce_forward + lce_backward) on the same inputs.

With 16-bit inputs and a chunk that holds the whole batch the call keeps the
logits instead of recomputing them; its logit gradient has the values the
recomputing backward forms, so lse, the loss scalars and d_weight must equal
the two-call results bit for bit, and d_hidden (summed over the vocabulary
in another grouping) must agree to fp32 rounding.  Other shapes take the
two-call algorithm inside the call.  Oracle tolerances as in test_gpu_ce.
"""
import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_amd import lce
from tests import synthetic as syn
from tests.test_gpu_ce import Case, _dev, _say, _sample, check_forward, check_grads, normwise

pytestmark = pytest.mark.gpu


def _single(c, chunk, grad_out=1.0, d_weight=None, accumulate=False):
    return lce.forward_backward(c.H, c.W, c.y, c.m, chunk=chunk, z_coef=c.z, grad_out=grad_out,
                                d_weight=d_weight, accumulate=accumulate)


def _workload(dt):
    import dataclasses
    return {"bf16": syn.QWEN_BF16, "f16": dataclasses.replace(syn.QWEN_BF16, dtype="f16"),
            "f64": syn.TINY_F64}[dt]


def _case(dt, *a, **k):
    c = Case(_workload(dt), *a, **k)
    if dt == "f16":
        c.w = syn.QWEN_BF16   # the 16-bit tolerances
    return c


KEPT = [
    # dtype, n, D, V, chunk, mask, z: the whole batch in one chunk (logits kept)
    ("bf16", 300, 192, 3000, 300, 0.05, 1e-4),   # ragged token and vocabulary tiles
    ("bf16", 517, 256, 2100, 600, None, 1e-3),   # chunk larger than the batch
    ("bf16", 1, 64, 33, 32, None, 0.0),          # one token: rows padded to 64 tokens
    ("bf16", 96, 128, 777, 96, 0.2, 0.0),
    ("bf16", 64, 64, 5000, 64, 0.25, 1e-2),
    ("f16", 300, 192, 3000, 300, 0.05, 1e-4),
    ("f16", 130, 128, 500, 132, None, 1e-3),
    ("bf16", 1028, 256, 5000, 1028, 0.05, 1e-4),  # three 512-token segments, the last ragged
    ("f16", 1540, 128, 3000, 1544, None, 1e-3),   # four segments, chunk past the batch
]


@pytest.mark.parametrize("dt,n,D,V,chunk,mask,z", KEPT)
def test_kept_logits_match_oracle_and_two_calls(dt, n, D, V, chunk, mask, z):
    _say(f"case {dt} n={n} D={D} V={V} chunk={chunk} mask={mask} z={z}")
    c = _case(dt, n, D, V, seed=n + 3 * D, mask_frac=mask, z=z)
    nb = lce.lce_forward_backward_workspace_bytes(n, D, V, chunk, c.H.dtype)
    assert nb > lce.lce_workspace_bytes(n, D, V, chunk, c.H.dtype)   # the logits are kept
    grad_out = 1024.0 if dt == "f16" else 1.5
    fwd, dH, dW = _single(c, chunk, grad_out=grad_out)
    torch.cuda.synchronize()
    ref = c.oracle_forward(chunk)
    check_forward(c, fwd, ref)
    rdH, rdW = oracle.backward(c.H64, c.W64, c.x.targets, ref["lse"], mask=c.x.mask, z_coef=c.z,
                               grad_out=grad_out)
    check_grads(c, dH, dW, rdH, rdW)
    # the two-call path on the same inputs
    f2 = c.gpu_forward(chunk)
    dH2, dW2 = c.gpu_backward(f2.lse, chunk, grad_out=grad_out)
    torch.cuda.synchronize()
    assert fwd.loss == f2.loss
    assert torch.equal(fwd.lse, f2.lse)
    assert torch.equal(dW, dW2)
    e = normwise(dH.double().cpu().numpy(), dH2.double().cpu().numpy())
    _say(f"  single vs two calls: d_hidden {e:.2e}")
    assert e <= 1e-2


OTHER = [
    # dtype, n, D, V, chunk, mask, z: the two-call algorithm inside the call
    ("bf16", 300, 192, 3000, 64, 0.05, 1e-4),    # chunk below the batch
    ("bf16", 96, 100, 777, 96, 0.2, 0.0),        # d_model % 8 != 0: generic core
    ("f64", 64, 64, 1000, 64, 0.25, 1e-4),       # fp64 inputs
]


@pytest.mark.parametrize("dt,n,D,V,chunk,mask,z", OTHER)
def test_other_shapes_match_oracle(dt, n, D, V, chunk, mask, z):
    _say(f"case {dt} n={n} D={D} V={V} chunk={chunk} mask={mask} z={z}")
    c = _case(dt, n, D, V, seed=n + D, mask_frac=mask, z=z)
    fwd, dH, dW = _single(c, chunk, grad_out=0.5)
    torch.cuda.synchronize()
    ref = c.oracle_forward(chunk)
    check_forward(c, fwd, ref)
    rdH, rdW = oracle.backward(c.H64, c.W64, c.x.targets, ref["lse"], mask=c.x.mask, z_coef=c.z,
                               grad_out=0.5)
    check_grads(c, dH, dW, rdH, rdW)


def test_accumulate_and_all_masked():
    c = Case(syn.QWEN_BF16, 200, 128, 1500, seed=31, mask_frac=0.1, z=1e-4)
    base = torch.randn(c.V, c.D, dtype=torch.float32, device=c.H.device)
    dw = base.clone()
    fwd, dH, dW = _single(c, 256, d_weight=dw, accumulate=True)
    _, dH1, dW1 = _single(c, 256)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH1)
    assert torch.equal(dW, base + dW1)
    c.m = torch.zeros(c.n, dtype=torch.uint8, device=c.H.device)
    fwd0, dH0, dW0 = _single(c, 256)
    torch.cuda.synchronize()
    assert fwd0.loss["n_counted"] == 0 and fwd0.loss["loss_mean"] == 0.0
    assert not dH0.any() and not dW0.any()


def test_refusals_leave_outputs_untouched():
    c = Case(syn.QWEN_BF16, 100, 64, 500, seed=5)
    dev = c.H.device
    lse = torch.full((c.n,), 7.0, device=dev)
    dh = torch.full_like(c.H, 3.0)
    dw = torch.full((c.V, c.D), 5.0, device=dev)
    nb = lce.lce_forward_backward_workspace_bytes(c.n, c.D, c.V, 128, c.H.dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    bad = c.y.clone()
    bad[37] = c.V
    st, _ = lce.lce_forward_backward(c.H, c.W, bad, None, c.n, c.D, c.V, 128, 0.0, 1.0, lse, dh,
                                     dw, 0, ws)
    assert st == 586
    short = ws[: nb - 257]
    st2, _ = lce.lce_forward_backward(c.H, c.W, c.y, None, c.n, c.D, c.V, 128, 0.0, 1.0, lse, dh,
                                      dw, 0, short)
    assert st2 == 582
    st3, _ = lce.lce_forward_backward(c.H, c.W, c.y, None, c.n, c.D, c.V, 128, float("nan"), 1.0,
                                      lse, dh, dw, 0, ws)
    assert st3 == 585
    torch.cuda.synchronize()
    assert bool((lse == 7.0).all()) and bool((dh == 3.0).all()) and bool((dw == 5.0).all())


def test_kept_logits_full_vocab():
    """256 tokens x 1024 x 151936 bf16 in one chunk of 256, 5% masked, z 1e-4
    (a shape where the call keeps the logits): sampled rows against the
    oracle, everything against the two-call path."""
    w = syn.QWEN_BF16
    _say("case 256 x 1024 x 151936 bf16, chunk 256: generating inputs")
    c = Case(w, 256, 1024, 151936, seed=41, mask_frac=0.05)
    assert lce.lce_forward_backward_keeps_logits(256, 1024, 151936, 256, c.H.dtype) == 1
    fwd, dH, dW = _single(c, 256)
    f2 = c.gpu_forward(256)
    dH2, dW2 = c.gpu_backward(f2.lse, 256)
    torch.cuda.synchronize()
    assert fwd.loss == f2.loss and torch.equal(fwd.lse, f2.lse) and torch.equal(dW, dW2)
    e = normwise(dH.double().cpu().numpy(), dH2.double().cpu().numpy())
    _say(f"  single vs two calls: d_hidden {e:.2e}")
    assert e <= 1e-2
    _say("  oracle forward (all tokens)")
    ref = c.oracle_forward(256)
    check_forward(c, fwd, ref)
    rng = np.random.default_rng(7)
    th = _sample(rng, c.n, 4)
    vw = np.unique(np.concatenate([_sample(rng, c.V, 4), c.x.targets[th]]))
    rdH = oracle.backward_dh_rows(c.H64, c.W64, c.x.targets, ref["lse"], th, mask=c.x.mask,
                                  z_coef=c.z)
    rdW = oracle.backward_dw_rows(c.H64, c.W64, c.x.targets, ref["lse"], vw, mask=c.x.mask,
                                  z_coef=c.z)
    check_grads(c, dH, dW, rdH, rdW, rows_h=th, rows_w=vw)


def test_kept_logits_full_size_512x4096():
    """512 x 4096 x 151936 bf16, chunk 512, z 1e-4, 5% masked (the single
    call's timed shape, where the cost model keeps the logits): lse, the loss
    and every d_hidden and d_weight element against the oracle, and lse, the
    loss scalars and d_weight bit for bit against the two-call path."""
    n, D, V, chunk = 512, 4096, 151936, 512
    _say(f"case kept logits full size {n} x {D} x {V}: generating inputs")
    c = _case("bf16", n, D, V, seed=7, mask_frac=0.05, z=1e-4)
    assert lce.lce_forward_backward_keeps_logits(n, D, V, chunk, c.H.dtype) == 1
    fwd, dH, dW = _single(c, chunk, grad_out=1.0)
    torch.cuda.synchronize()
    _say("  oracle forward (all tokens)")
    ref = c.oracle_forward(chunk)
    check_forward(c, fwd, ref)
    _say("  oracle backward: every d_hidden and d_weight element")
    rdH, rdW = oracle.backward(c.H64, c.W64, c.x.targets, ref["lse"], mask=c.x.mask, z_coef=c.z,
                               grad_out=1.0)
    check_grads(c, dH, dW, rdH, rdW)
    del rdH, rdW
    f2 = c.gpu_forward(chunk)
    dH2, dW2 = c.gpu_backward(f2.lse, chunk, grad_out=1.0)
    torch.cuda.synchronize()
    assert fwd.loss == f2.loss
    assert torch.equal(fwd.lse, f2.lse)
    assert torch.equal(dW, dW2)
    e = normwise(dH.double().cpu().numpy(), dH2.double().cpu().numpy())
    _say(f"  single vs two calls: d_hidden {e:.2e}")
    assert e <= 1e-2
