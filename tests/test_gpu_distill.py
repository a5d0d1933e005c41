"""GPU parity of lce_distill_fwd_bwd (distillation + z-loss) against the CPU
fp64 oracle, through the C ABI.  bf16/fp32: loss relative error <= 2e-3,
gradient max|diff| <= 1e-2 * max|ref|; fp64: 1e-10 for both."""
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
@pytest.mark.parametrize("obj", [0, 1, 2])
@pytest.mark.parametrize("n,V", [(37, 1000), (20, 1003), (4, 151936),
                                 # the largest vocabulary whose student rows fit the
                                 # registers, and the next multiple of 8 (streamed rows)
                                 (2, 155648), (3, 155656)])
def test_small_distill(dt, obj, n, V):
    print(f"case distill {dt} obj={obj} n={n} V={V}", flush=True)
    dev = _dev()
    d = syn.distill_inputs(syn.DISTILL_BF16, n_tok=n, vocab=V, seed=n + obj, dtype=dt)
    S, U = d.student.to(dev), d.teacher.to(dev)
    m = torch.from_numpy(d.mask).to(dev)
    out, g = lce.distill(S, U, m, objective=obj, temperature=2.0, z_coef=1e-3, grad_out=1.3)
    r = oracle.distill(d.student.double().numpy(), d.teacher.double().numpy(), mask=d.mask,
                       objective=obj, temperature=2.0, z_coef=1e-3, grad_out=1.3)
    lt, gt = TOL[dt]
    assert out["n_counted"] == r["n_counted"]
    el = abs(out["loss_mean"] - r["loss"]) / abs(r["loss"])
    ez = abs(out["z_mean"] - r["z_loss"]) / abs(r["z_loss"])
    eg = normwise(g.double().cpu().numpy(), r["grad"])
    print(f"  loss rel {el:.2e} z rel {ez:.2e} grad {eg:.2e}", flush=True)
    assert el <= lt and ez <= lt and eg <= gt
    assert not g[m == 0].any()


@pytest.mark.parametrize("obj", [0, 1, 2])
@pytest.mark.parametrize("n,V", [(37, 1000), (3, 155656)])
@pytest.mark.parametrize("grad_out,z,shift", [(-0.7, 1e-3, 0.0), (1.3, 0.5, -40.0)])
def test_negative_gradient_scale(obj, n, V, grad_out, z, shift):
    """The gradient's terms with negative coefficients: grad_out < 0 (every
    term), and 1 + 2 z lse_student < 0 (student logits shifted down by 40 with
    z 0.5; objectives 0 and 1), bf16 rows resident (V 1000) and streamed."""
    print(f"case distill sign obj={obj} n={n} V={V} g={grad_out} z={z} shift={shift}", flush=True)
    dev = _dev()
    d = syn.distill_inputs(syn.DISTILL_BF16, n_tok=n, vocab=V, seed=70 + obj + n, dtype="bf16")
    S = (d.student.float() + shift).to(torch.bfloat16)
    U = d.teacher
    m = torch.from_numpy(d.mask)
    out, g = lce.distill(S.to(dev), U.to(dev), m.to(dev), objective=obj, temperature=2.0,
                         z_coef=z, grad_out=grad_out)
    r = oracle.distill(S.double().numpy(), U.double().numpy(), mask=d.mask, objective=obj,
                       temperature=2.0, z_coef=z, grad_out=grad_out)
    el = abs(out["loss_mean"] - r["loss"]) / abs(r["loss"])
    ez = abs(out["z_mean"] - r["z_loss"]) / abs(r["z_loss"])
    eg = normwise(g.double().cpu().numpy(), r["grad"])
    print(f"  loss rel {el:.2e} z rel {ez:.2e} grad {eg:.2e}", flush=True)
    assert el <= 2e-3 and ez <= 2e-3 and eg <= 1e-2


@pytest.mark.parametrize("obj", [0, 1, 2])
def test_f16_distill(obj):
    """fp16 logits; grad_out carries a loss scale as in fp16 training."""
    dev = _dev()
    n, V = 37, 1000
    d = syn.distill_inputs(syn.DISTILL_BF16, n_tok=n, vocab=V, seed=60 + obj, dtype="f16")
    S, U = d.student.to(dev), d.teacher.to(dev)
    assert S.dtype == torch.float16
    m = torch.from_numpy(d.mask).to(dev)
    out, g = lce.distill(S, U, m, objective=obj, temperature=2.0, z_coef=1e-3, grad_out=1024.0)
    r = oracle.distill(d.student.double().numpy(), d.teacher.double().numpy(), mask=d.mask,
                       objective=obj, temperature=2.0, z_coef=1e-3, grad_out=1024.0)
    el = abs(out["loss_mean"] - r["loss"]) / abs(r["loss"])
    ez = abs(out["z_mean"] - r["z_loss"]) / abs(r["z_loss"])
    eg = normwise(g.double().cpu().numpy(), r["grad"])
    print(f"  f16 obj {obj}: loss rel {el:.2e} z rel {ez:.2e} grad {eg:.2e}", flush=True)
    assert g.dtype == torch.float16
    assert el <= 2e-3 and ez <= 2e-3 and eg <= 1e-2


@pytest.mark.parametrize("obj", [1, 2])
def test_kl_zero_for_identical_logits(obj):
    dev = _dev()
    d = syn.distill_inputs(syn.DISTILL_BF16, n_tok=16, vocab=512, seed=3)
    S = d.student.to(dev)
    out, g = lce.distill(S, S.clone(), None, objective=obj, temperature=2.0)
    assert abs(out["loss_mean"]) <= 1e-6
    assert float(g.float().abs().max()) <= 1e-6


def test_distill_refusals():
    dev = _dev()
    d = syn.distill_inputs(syn.DISTILL_BF16, n_tok=8, vocab=64, seed=4)
    S, U = d.student.to(dev), d.teacher.to(dev)
    g = torch.full_like(S, 9.0)
    ws = torch.empty(lce.lce_distill_workspace_bytes(8, 64), dtype=torch.uint8, device=dev)
    call = lambda **kw: lce.lce_distill_fwd_bwd(**{**dict(
        student=S, teacher=U, loss_mask=None, n_tok=8, vocab=64, objective=0, temperature=1.0,
        z_coef=0.0, grad_out=1.0, grad_logits=g, workspace=ws), **kw})[0]
    assert call(objective=3) == 588
    assert call(temperature=0.0) == 585
    assert call(temperature=float("nan")) == 585
    assert call(teacher=U.float()) == 590
    assert call(grad_logits=g[:4]) == 582
    assert call(n_tok=0) == 581
    torch.cuda.synchronize()
    assert torch.all(g == 9.0)


@pytest.mark.parametrize("obj", [0, 1, 2])
@pytest.mark.parametrize("n,V", [(37, 1000), (3, 155656)])
def test_async_distill_matches_sync(obj, n, V):
    """lce_distill_fwd_bwd without a host result returns once enqueued; the
    gradient it writes and the scalars lce_loss_fetch then returns equal the
    synchronous call's bit for bit.  The allocation-free call has no
    workspace to fetch from and refuses a NULL result with 582."""
    print(f"case async distill obj={obj} n={n} V={V}", flush=True)
    dev = _dev()
    d = syn.distill_inputs(syn.DISTILL_BF16, n_tok=n, vocab=V, seed=90 + obj, dtype="bf16")
    S, U = d.student.to(dev), d.teacher.to(dev)
    m = torch.from_numpy(d.mask).to(dev)
    nb = lce.lce_distill_workspace_bytes(n, V)
    ws1 = torch.empty(nb, dtype=torch.uint8, device=dev)
    ws2 = torch.empty(nb, dtype=torch.uint8, device=dev)
    g1 = torch.empty_like(S)
    g2 = torch.full_like(S, 5.0)
    args = dict(student=S, teacher=U, loss_mask=m, n_tok=n, vocab=V, objective=obj,
                temperature=2.0, z_coef=1e-3, grad_out=1.3)
    st, ref = lce.lce_distill_fwd_bwd(**args, grad_logits=g1, workspace=ws1)
    assert st == 580
    st, out = lce.lce_distill_fwd_bwd(**args, grad_logits=g2, workspace=ws2, sync=False)
    assert st == 580 and out is None
    st, loss = lce.lce_loss_fetch(ws2)
    assert st == 580
    assert loss.as_dict() == ref.as_dict()
    assert torch.equal(g1, g2)
    L = lce.lib()
    ts = [lce._t(S), lce._t(U), lce._t(m), lce._t(g2)]
    st = L.lce_distill_fwd_bwd_noalloc(*[lce.ctypes.byref(a) for a in ts[:3]], n, V, obj, 2.0,
                                       1e-3, 1.3, lce.ctypes.byref(ts[3]), None,
                                       lce._stream(dev))
    assert st == 582


def test_distill_full_size_sampled_rows():
    """4096 x 151936 bf16, T = 2, 10% masked, z 1e-4: every objective."""
    w = syn.DISTILL_BF16
    dev = _dev()
    print(f"case {w.name}: generating inputs", flush=True)
    d = syn.distill_inputs(w)
    S, U = d.student.to(dev), d.teacher.to(dev)
    m = torch.from_numpy(d.mask).to(dev)
    C = int(d.mask.sum())
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, w.n_tok - 1], rng.choice(w.n_tok, 10, replace=False),
                                     np.flatnonzero(d.mask == 0)[:2]]))
    S64, U64 = d.student.double().numpy(), d.teacher.double().numpy()
    for obj in (0, 1, 2):
        out, g = lce.distill(S, U, m, objective=obj, temperature=w.temperature, z_coef=w.z_coef)
        torch.cuda.synchronize()
        full = oracle.distill(S64, U64, mask=d.mask, objective=obj, temperature=w.temperature,
                              z_coef=w.z_coef, want_grad=False)
        el = abs(out["loss_mean"] - full["loss"]) / abs(full["loss"])
        ez = abs(out["z_mean"] - full["z_loss"]) / abs(full["z_loss"])
        print(f"  objective {obj}: loss rel {el:.2e} z rel {ez:.2e}", flush=True)
        assert el <= 2e-3 and ez <= 2e-3
        gr, rl, rz = oracle.distill_rows(d.student[rows].double().numpy(),
                                         d.teacher[rows].double().numpy(), C,
                                         row_mask=d.mask[rows], objective=obj,
                                         temperature=w.temperature, z_coef=w.z_coef)
        eg = normwise(g[torch.from_numpy(rows).to(dev)].double().cpu().numpy(), gr)
        assert out["n_counted"] == C
        print(f"  objective {obj}: loss {out['loss_mean']:.6g} z {out['z_mean']:.6g} "
              f"sampled grad {eg:.2e}", flush=True)
        assert eg <= 1e-2
