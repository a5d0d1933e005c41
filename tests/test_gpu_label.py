"""GPU parity of lce_ce_logits_fwd_bwd (label cross-entropy + z-loss from
materialized logits) against the CPU fp64 oracle, through the C ABI.
bf16/fp32: loss relative error <= 2e-3, gradient max|diff| <= 1e-2 * max|ref|;
fp64: 1e-10 for both."""
import math

import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_amd import lce
from tests import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = {"bf16": (2e-3, 1e-2), "f32": (2e-3, 1e-2), "f64": (1e-10, 1e-10)}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def normwise(a, ref):
    return float(np.max(np.abs(a - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


@pytest.mark.parametrize("dt", ["bf16", "f32", "f64"])
@pytest.mark.parametrize("n,V,mask_frac", [(37, 1000, 0.2), (20, 1003, 0.0), (3, 4096, 0.34),
                                            (5, 151936, 0.2), (3, 155648, 0.0),
                                            (3, 155656, 0.0)])   # rows past the registers
def test_small_label_ce(dt, n, V, mask_frac):
    print(f"case label {dt} n={n} V={V} mask {mask_frac}", flush=True)
    dev = _dev()
    w = syn.LabelWorkload("small", n, V, dt, 1e-3, mask_frac, 40 + n)
    d = syn.label_inputs(w)
    Z = d.logits.to(dev)
    y = torch.from_numpy(d.targets).to(dev)
    m = torch.from_numpy(d.mask).to(dev) if d.mask is not None else None
    out, g = lce.ce_logits(Z, y, m, z_coef=1e-3, grad_out=1.3)
    r = oracle.ce_logits(d.logits.double().numpy(), d.targets, mask=d.mask, z_coef=1e-3,
                         grad_out=1.3)
    lt, gt = TOL[dt]
    assert out["n_counted"] == r["n_counted"]
    el = abs(out["loss_mean"] - r["loss"]) / abs(r["loss"])
    ez = abs(out["z_mean"] - r["z_loss"]) / abs(r["z_loss"])
    eg = normwise(g.double().cpu().numpy(), r["grad"])
    print(f"  loss rel {el:.2e} z rel {ez:.2e} grad {eg:.2e}", flush=True)
    assert el <= lt and ez <= lt and eg <= gt
    if m is not None:
        assert not g[m == 0].any()
    # loss only: the same scalars without a gradient pass (16-bit rows that fit
    # the registers take another kernel with another summation order)
    out2, g2 = lce.ce_logits(Z, y, m, z_coef=1e-3, grad_out=1.3, want_grad=False)
    assert g2 is None
    rt = 1e-6 if dt == "bf16" else 0.0
    assert abs(out2["loss_sum"] - out["loss_sum"]) <= rt * abs(out["loss_sum"])
    assert abs(out2["z_sum"] - out["z_sum"]) <= rt * abs(out["z_sum"])


@pytest.mark.parametrize("n,V", [(37, 1000), (3, 155656)])
@pytest.mark.parametrize("grad_out,z,shift", [(-0.7, 1e-3, 0.0), (1.3, 0.5, -20.0)])
def test_negative_gradient_scale(n, V, grad_out, z, shift):
    """g (1 + 2 z lse) < 0: grad_out < 0, and lse < -1/(2 z) (logits shifted
    down by 20 with z 0.5), bf16 rows in registers (V 1000) and streamed."""
    print(f"case label sign n={n} V={V} g={grad_out} z={z} shift={shift}", flush=True)
    dev = _dev()
    w = syn.LabelWorkload("sign", n, V, "bf16", z, 0.2, 80 + n)
    d = syn.label_inputs(w)
    Z = (d.logits.float() + shift).to(torch.bfloat16)
    m = torch.from_numpy(d.mask) if d.mask is not None else None
    out, g = lce.ce_logits(Z.to(dev), torch.from_numpy(d.targets).to(dev),
                           m.to(dev) if m is not None else None, z_coef=z, grad_out=grad_out)
    r = oracle.ce_logits(Z.double().numpy(), d.targets, mask=d.mask, z_coef=z, grad_out=grad_out)
    el = abs(out["loss_mean"] - r["loss"]) / abs(r["loss"])
    ez = abs(out["z_mean"] - r["z_loss"]) / abs(r["z_loss"])
    eg = normwise(g.double().cpu().numpy(), r["grad"])
    print(f"  loss rel {el:.2e} z rel {ez:.2e} grad {eg:.2e}", flush=True)
    assert el <= 2e-3 and ez <= 2e-3 and eg <= 1e-2


@pytest.mark.parametrize("n,V", [(37, 1000), (20, 1003)])
def test_f16_label_ce(n, V):
    """fp16 logits; grad_out carries a loss scale as in fp16 training."""
    dev = _dev()
    w = syn.LabelWorkload("small_f16", n, V, "f16", 1e-3, 0.2, 80 + n)
    d = syn.label_inputs(w)
    Z = d.logits.to(dev)
    assert Z.dtype == torch.float16
    y = torch.from_numpy(d.targets).to(dev)
    m = torch.from_numpy(d.mask).to(dev)
    out, g = lce.ce_logits(Z, y, m, z_coef=1e-3, grad_out=1024.0)
    r = oracle.ce_logits(d.logits.double().numpy(), d.targets, mask=d.mask, z_coef=1e-3,
                         grad_out=1024.0)
    el = abs(out["loss_mean"] - r["loss"]) / abs(r["loss"])
    ez = abs(out["z_mean"] - r["z_loss"]) / abs(r["z_loss"])
    eg = normwise(g.double().cpu().numpy(), r["grad"])
    print(f"  f16 label: loss rel {el:.2e} z rel {ez:.2e} grad {eg:.2e}", flush=True)
    assert el <= 2e-3 and ez <= 2e-3 and eg <= 1e-2


def test_uniform_logits_give_log_vocab():
    dev = _dev()
    n, V = 5, 151936
    Z = torch.zeros(n, V, dtype=torch.bfloat16, device=dev)
    y = torch.tensor([0, 1, V // 2, V - 2, V - 1], device=dev)
    out, g = lce.ce_logits(Z, y)
    assert abs(out["loss_mean"] - math.log(V)) <= 2e-3 * math.log(V)
    want = np.full((n, V), 1.0 / (n * V))
    want[np.arange(n), y.cpu().numpy()] -= 1.0 / n
    assert normwise(g.double().cpu().numpy(), want) <= 1e-2


def test_label_refusals_leave_outputs_untouched():
    dev = _dev()
    d = syn.label_inputs(syn.LABEL_BF16, n_tok=8, vocab=64, seed=7)
    Z = d.logits.to(dev)
    y = torch.from_numpy(d.targets).to(dev)
    g = torch.full_like(Z, 9.0)
    ws = torch.empty(lce.lce_distill_workspace_bytes(8, 64), dtype=torch.uint8, device=dev)
    call = lambda **kw: lce.lce_ce_logits_fwd_bwd(**{**dict(
        logits=Z, targets=y, loss_mask=None, n_tok=8, vocab=64, z_coef=0.0, grad_out=1.0,
        grad_logits=g, workspace=ws), **kw})[0]
    bad = y.clone()
    bad[5] = 64
    assert call(targets=bad) == 586
    bad[5] = -1
    assert call(targets=bad) == 586
    assert call(z_coef=float("nan")) == 585
    assert call(grad_logits=g.float()) == 590
    assert call(targets=y.int()) == 590
    assert call(grad_logits=g[:4]) == 582
    assert call(workspace=ws[:64]) == 582
    assert call(n_tok=0) == 581
    torch.cuda.synchronize()
    assert torch.all(g == 9.0)
    assert call() == 580


@pytest.mark.parametrize("n,V,grad", [(37, 1000, True), (3, 155656, True), (20, 1003, False)])
def test_async_label_ce(n, V, grad):
    """lce_ce_logits_fwd_bwd without a host result returns once enqueued: its
    gradient and the scalars lce_loss_fetch then returns equal the
    synchronous call's bit for bit; a target out of range shows as 586 in
    lce_loss_fetch and leaves the gradient untouched."""
    print(f"case async label CE n={n} V={V} grad={grad}", flush=True)
    dev = _dev()
    d = syn.label_inputs(syn.LABEL_BF16, n_tok=n, vocab=V, seed=31 + n)
    Z = d.logits.to(dev)
    y = torch.from_numpy(d.targets).to(dev)
    m = torch.from_numpy(d.mask).to(dev) if d.mask is not None else None
    nb = lce.lce_distill_workspace_bytes(n, V)
    ws1 = torch.empty(nb, dtype=torch.uint8, device=dev)
    ws2 = torch.empty(nb, dtype=torch.uint8, device=dev)
    g1 = torch.empty_like(Z) if grad else None
    g2 = torch.full_like(Z, 3.0) if grad else None
    args = dict(logits=Z, targets=y, loss_mask=m, n_tok=n, vocab=V, z_coef=1e-3, grad_out=0.8)
    st, ref = lce.lce_ce_logits_fwd_bwd(**args, grad_logits=g1, workspace=ws1)
    assert st == 580
    st, out = lce.lce_ce_logits_fwd_bwd(**args, grad_logits=g2, workspace=ws2, sync=False)
    assert st == 580 and out is None
    st, loss = lce.lce_loss_fetch(ws2)
    assert st == 580
    assert loss.as_dict() == ref.as_dict()
    if grad:
        assert torch.equal(g1, g2)
    bad = y.clone()
    bad[n // 2] = V
    g3 = torch.full_like(Z, 7.0) if grad else None
    st, _ = lce.lce_ce_logits_fwd_bwd(**{**args, "targets": bad}, grad_logits=g3, workspace=ws2,
                                      sync=False)
    assert st == 580                                  # enqueued; the verdict is fetched
    assert lce.lce_loss_fetch(ws2)[0] == 586
    if grad:
        assert torch.all(g3 == 7.0)


def test_label_ce_full_size_sampled_rows():
    """4096 x 151936 bf16 logits, 10% masked, z 1e-4: the loss of every row
    and the gradient of sampled rows against the oracle."""
    w = syn.LABEL_BF16
    dev = _dev()
    print(f"case {w.name}: generating inputs", flush=True)
    d = syn.label_inputs(w)
    Z = d.logits.to(dev)
    y = torch.from_numpy(d.targets).to(dev)
    m = torch.from_numpy(d.mask).to(dev)
    out, g = lce.ce_logits(Z, y, m, z_coef=w.z_coef)
    torch.cuda.synchronize()
    Z64 = d.logits.double().numpy()
    full = oracle.ce_logits(Z64, d.targets, mask=d.mask, z_coef=w.z_coef, want_grad=False)
    el = abs(out["loss_mean"] - full["loss"]) / abs(full["loss"])
    ez = abs(out["z_mean"] - full["z_loss"]) / abs(full["z_loss"])
    print(f"  loss {out['loss_mean']:.6g} rel {el:.2e} z rel {ez:.2e}", flush=True)
    assert out["n_counted"] == full["n_counted"]
    assert el <= 2e-3 and ez <= 2e-3
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, w.n_tok - 1], rng.choice(w.n_tok, 10, replace=False),
                                     np.flatnonzero(d.mask == 0)[:2]]))
    gr, rl, rz = oracle.ce_logits_rows(Z64[rows], d.targets[rows], full["n_counted"],
                                       row_mask=d.mask[rows], z_coef=w.z_coef)
    eg = normwise(g[torch.from_numpy(rows).to(dev)].double().cpu().numpy(), gr)
    print(f"  sampled grad {eg:.2e}", flush=True)
    assert eg <= 1e-2
