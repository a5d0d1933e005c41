"""GPU parity of the fused path at the method's edge cases, against the CPU fp64
oracle and against closed forms, through the C ABI.

* A negative logit-gradient coefficient.  The per-token coefficient of the
  softmax term, grad_out/C * (1 + 2 z_coef lse_t) (Fast-LLM 566, "What it
  does"), is negative when grad_out < 0, or with z-loss when
  lse_t < -1/(2 z_coef).  The 16-bit epilogues fold |coef| into the exponent
  and apply its sign separately; these cases drive that branch through
  lce_backward, the single call that keeps the logits, and the vocabulary-shard
  backward.
* The lossk page's worked example, "A worked example: uniform logits give
  exactly log(vocab)", on the fused path: W = 0 makes every logit exactly 0,
  so every token's loss is ln V, its z-loss (ln V)^2, d_hidden = d W is exactly
  zero and d_weight has the closed form
      d_weight[v] = sum_t m_t (c_t / V) H_t - sum_{t: y_t = v} m_t g H_t,
      c_t = g + 2 g_z ln V,  g = grad_out / C,  g_z = z_coef g.
* Logits of magnitude 10^2-10^3 (large W), where the online max shift and the
  folded exponent carry the whole range.
* The z-loss identities of Fast-LLM 566 ("What it does", "Changes"): the
  forward does not depend on z_coef; the gradient with z on equals the
  gradient with z off plus the z-only term; with z off the vocabulary sum of
  d_weight cancels, with z on it equals sum_t 2 g_z lse_t H_t.

Tolerances: fp64 1e-10 (loss relative, gradients max|diff| / max|ref|);
bf16 / fp16 2e-3 and 1e-2; closed forms as stated per test.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_amd import lce
from tests import synthetic as syn
from tests.test_gpu_ce import Case, _dev, _say, check_forward, check_grads, normwise
from tests.test_gpu_shard import run_shards

pytestmark = pytest.mark.gpu

F16 = dataclasses.replace(syn.QWEN_BF16, dtype="f16")


def _workload(dt):
    return {"bf16": syn.QWEN_BF16, "f16": F16, "f64": syn.TINY_F64}[dt]


def _case(dt, n, D, V, seed, mask=None, z=0.0):
    c = Case(_workload(dt), n, D, V, seed=seed, mask_frac=mask, z=z)
    if dt == "f16":
        c.w = syn.QWEN_BF16            # the 16-bit tolerances
    return c


def _rebuild(c):
    """Device copies and fp64 views after the CPU inputs were edited."""
    dev = _dev()
    c.H = c.x.hidden.to(dev)
    c.W = c.x.weight.to(dev)
    c.H64, c.W64 = c.x.hidden64(), c.x.weight64()
    return c


def _biased(c, bias=20.0, lo=0.25, seed=0):
    """Feature 0 of every token set to lo or 1 (seeded) and column 0 of W to
    -bias: the logits sit near -bias * h0, so tokens with h0 = 1 get
    lse ~ -bias + ln V (strongly negative) and the others a positive lse."""
    rng = np.random.default_rng(seed)
    h0 = np.where(rng.random(c.n) < 0.5, lo, 1.0)
    c.x.hidden[:, 0] = torch.from_numpy(h0).to(c.x.hidden.dtype)
    c.x.weight[:, 0] = -bias
    return _rebuild(c)


def _coef_factor(ref_lse, z):
    return 1.0 + 2.0 * z * np.asarray(ref_lse)


def _oracle_grads(c, lse, grad_out):
    return oracle.backward(c.H64, c.W64, c.x.targets, lse, mask=c.x.mask, z_coef=c.z,
                           grad_out=grad_out)


# --------------------------------------------------- negative coefficient --

NEG = [
    # dtype, n, D, V, chunk, mask, z, grad_out, biased
    ("bf16", 300, 192, 3000, 64, 0.05, 1e-4, -1.5, False),    # grad_out < 0
    ("bf16", 517, 256, 5000, 256, None, 1e-3, -0.75, False),  # slab pipeline, several slabs
    ("f16", 300, 192, 3000, 64, 0.05, 1e-4, -1024.0, False),
    ("f64", 64, 64, 1000, 16, 0.25, 1e-4, -2.0, False),
    ("bf16", 300, 192, 3000, 64, 0.1, 0.1, 1.0, True),        # lse < -1/(2 z) for half the tokens
    ("bf16", 1100, 64, 40000, 1100, 0.05, 0.1, 1.0, True),    # shorter first slab
    ("f16", 300, 128, 3000, 64, 0.1, 0.1, 256.0, True),
    ("f64", 70, 64, 1000, 16, 0.1, 0.1, 1.0, True),
    ("bf16", 300, 192, 3000, 64, 0.1, 0.1, -1.0, True),       # both signs flipped
]


@pytest.mark.parametrize("dt,n,D,V,chunk,mask,z,g,biased", NEG)
def test_negative_coefficient_two_calls(dt, n, D, V, chunk, mask, z, g, biased):
    _say(f"case neg-coef {dt} n={n} D={D} V={V} chunk={chunk} z={z} grad_out={g} "
         f"biased={biased}")
    c = _case(dt, n, D, V, seed=n + V, mask=mask, z=z)
    if biased:
        _biased(c, seed=n)
    fwd = c.gpu_forward(chunk)
    ref = c.oracle_forward(chunk)
    check_forward(c, fwd, ref)
    f = g * _coef_factor(ref["lse"], z)
    counted = np.ones(n, bool) if c.x.mask is None else c.x.mask.astype(bool)
    _say(f"  coefficient sign: {int((f[counted] < 0).sum())} negative, "
         f"{int((f[counted] > 0).sum())} positive of {int(counted.sum())} counted tokens")
    assert (f[counted] < 0).any()
    if biased:
        assert (f[counted] > 0).any()
    dH, dW = c.gpu_backward(fwd.lse, chunk, grad_out=g)
    rdH, rdW = _oracle_grads(c, ref["lse"], g)
    check_grads(c, dH, dW, rdH, rdW)


KEPT_NEG = [
    # dtype, n, D, V, chunk, mask, z, grad_out, biased
    ("bf16", 200, 128, 3000, 256, 0.05, 1e-4, -1.5, False),
    ("bf16", 200, 128, 3000, 256, 0.1, 0.1, 1.0, True),
    ("f16", 130, 128, 2000, 132, 0.1, 0.1, 512.0, True),
    ("f16", 130, 128, 2000, 132, None, 1e-3, -1024.0, False),
]


@pytest.mark.parametrize("dt,n,D,V,chunk,mask,z,g,biased", KEPT_NEG)
def test_negative_coefficient_kept_logits(dt, n, D, V, chunk, mask, z, g, biased):
    """lce_forward_backward on shapes where it keeps the logits: the
    logit-gradient pass over the kept logits takes the sign branch."""
    _say(f"case neg-coef kept {dt} n={n} D={D} V={V} chunk={chunk} z={z} grad_out={g}")
    c = _case(dt, n, D, V, seed=3 * n + V, mask=mask, z=z)
    if biased:
        _biased(c, seed=n + 1)
    assert lce.lce_forward_backward_keeps_logits(n, D, V, chunk, c.H.dtype) == 1
    fwd, dH, dW = lce.forward_backward(c.H, c.W, c.y, c.m, chunk=chunk, z_coef=z, grad_out=g)
    torch.cuda.synchronize()
    ref = c.oracle_forward(chunk)
    check_forward(c, fwd, ref)
    f = g * _coef_factor(ref["lse"], z)
    assert (f < 0).any()
    rdH, rdW = _oracle_grads(c, ref["lse"], g)
    check_grads(c, dH, dW, rdH, rdW)


SHARD_NEG = [
    # dtype, n, D, V, bounds, chunk, mask, z, grad_out, biased
    ("bf16", 300, 128, 3000, [0, 1024, 1100, 3000], 64, 0.05, 1e-4, -1.25, False),
    ("bf16", 257, 256, 5000, [0, 1280, 2560, 5000], 256, 0.1, 0.1, 1.0, True),
    ("f64", 70, 64, 1000, [0, 300, 1000], 16, 0.2, 0.1, 1.0, True),
]


@pytest.mark.parametrize("dt,n,D,V,bounds,chunk,mask,z,g,biased", SHARD_NEG)
def test_negative_coefficient_shards(dt, n, D, V, bounds, chunk, mask, z, g, biased):
    _say(f"case neg-coef shards {dt} n={n} D={D} V={V} bounds={bounds} z={z} grad_out={g}")
    c = _case(dt, n, D, V, seed=n + 7 * V, mask=mask, z=z)
    if biased:
        _biased(c, seed=n + 2)
    out, lse, _, dH, dW = run_shards(c.H, c.W, c.y, c.m, bounds, chunk, z, grad_out=g)
    ref = c.oracle_forward(chunk)
    lt, gt = (1e-10, 1e-10) if dt == "f64" else (2e-3, 1e-2)
    e = abs(out["loss_mean"] - ref["loss_mean"]) / abs(ref["loss_mean"])
    assert e <= lt and normwise(lse.double().cpu().numpy(), ref["lse"]) <= lt
    f = g * _coef_factor(ref["lse"], z)
    assert (f < 0).any()
    rdH, rdW = _oracle_grads(c, ref["lse"], g)
    eh = normwise(dH.cpu().numpy(), rdH)
    ew = normwise(dW.double().cpu().numpy(), rdW)
    _say(f"  loss rel {e:.2e}; dH {eh:.2e} dW {ew:.2e}")
    assert eh <= gt and ew <= gt


# ------------------------------------------ uniform logits: W = 0, ln V --

ZERO_W = [
    # dtype, n, D, V, chunk, mask, z, grad_out
    ("f64", 64, 64, 1000, 16, 0.25, 1e-3, 1.0),
    ("bf16", 200, 128, 1000, 64, 0.1, 1e-3, 1.0),
    ("f64", 48, 64, 151936, 16, 0.25, 1e-2, 1.5),
    ("bf16", 300, 128, 151936, 256, 0.05, 1e-2, 1.0),
    ("f16", 300, 128, 151936, 256, 0.05, 1e-2, 1024.0),
]


@pytest.mark.parametrize("dt,n,D,V,chunk,mask,z,g", ZERO_W)
def test_zero_weight_gives_ln_vocab(dt, n, D, V, chunk, mask, z, g):
    _say(f"case W=0 {dt} n={n} D={D} V={V} chunk={chunk} z={z}")
    c = _case(dt, n, D, V, seed=n + D, mask=mask, z=z)
    c.x.weight.zero_()
    _rebuild(c)
    fwd = c.gpu_forward(chunk)
    dH, dW = c.gpu_backward(fwd.lse, chunk, grad_out=g)
    torch.cuda.synchronize()
    lnV = math.log(V)
    # exact arithmetic: every lse is log(V) up to one rounding of log in the
    # accumulator type (fp32 on the 16-bit paths)
    rtol = 1e-13 if dt == "f64" else 1e-6
    eloss = abs(fwd.loss["loss_mean"] - lnV) / lnV
    ez = abs(fwd.loss["z_mean"] - lnV * lnV) / (lnV * lnV)
    else_ = float(np.max(np.abs(fwd.lse.double().cpu().numpy() - lnV))) / lnV
    _say(f"  loss {fwd.loss['loss_mean']!r} vs ln V {lnV!r} (rel {eloss:.1e}); z rel {ez:.1e}; "
         f"lse {else_:.1e}")
    assert eloss <= rtol and ez <= 2 * rtol and else_ <= rtol
    assert not dH.any()                      # d W with W = 0 is exactly zero
    # d_weight against the closed form (fp64, from the inputs only)
    H = c.H64
    m = np.ones(n) if c.x.mask is None else c.x.mask.astype(np.float64)
    C = m.sum()
    gg, gz = g / C, z * g / C
    coef = gg + 2.0 * gz * lnV
    ref = np.tile((m * coef / V) @ H, (V, 1))
    np.add.at(ref, c.x.targets, -(m * gg)[:, None] * H)
    gtol = 1e-10 if dt == "f64" else 1e-2
    ew = normwise(dW.double().cpu().numpy(), ref)
    # the vocabulary sum of d_weight: sum_t m_t 2 g_z ln V H_t (0 without z)
    colsum = dW.double().sum(0).cpu().numpy()
    ref_cs = (m * 2.0 * gz * lnV) @ H
    ecs = float(np.max(np.abs(colsum - ref_cs))) / max(float(np.max(np.abs(dW.double().cpu().numpy()))), 1e-300)
    _say(f"  d_weight vs closed form {ew:.2e}; vocabulary sum {ecs:.2e}")
    assert ew <= gtol
    assert ecs <= (1e-9 if dt == "f64" else 5e-2)


# ----------------------------------------------------------- large logits --

LARGE = [
    # dtype, n, D, V, chunk, sigma_w, mask, z: logit std = sigma_w * sqrt(D)
    ("f64", 64, 64, 1000, 16, 40.0, 0.25, 1e-4),        # std 320
    ("f64", 64, 64, 1000, 16, 2.0, None, 1e-3),          # std 16
    ("bf16", 300, 256, 3000, 64, 20.0, 0.05, 1e-4),     # std 320
    ("bf16", 300, 256, 3000, 64, 4.0, None, 1e-3),      # std 64
    ("bf16", 1100, 64, 40000, 1100, 60.0, 0.05, 1e-4),  # std 480, shorter first slab
    ("f16", 300, 256, 3000, 64, 10.0, 0.05, 1e-4),      # std 160 (fp16 holds |W| < 65504)
]


@pytest.mark.parametrize("dt,n,D,V,chunk,sw,mask,z", LARGE)
def test_large_magnitude_logits(dt, n, D, V, chunk, sw, mask, z):
    _say(f"case large logits {dt} n={n} D={D} V={V} sigma_w={sw} (logit std "
         f"{sw * math.sqrt(D):.0f})")
    w = dataclasses.replace(_workload(dt), sigma_w=sw)
    c = Case(w, n, D, V, seed=n + 11, mask_frac=mask, z=z)
    if dt == "f16":
        c.w = syn.QWEN_BF16
    fwd = c.gpu_forward(chunk)
    ref = c.oracle_forward(chunk)
    _say(f"  oracle lse range [{ref['lse'].min():.1f}, {ref['lse'].max():.1f}]")
    check_forward(c, fwd, ref)
    g = 1024.0 if dt == "f16" else 1.0
    dH, dW = c.gpu_backward(fwd.lse, chunk, grad_out=g)
    rdH, rdW = _oracle_grads(c, ref["lse"], g)
    check_grads(c, dH, dW, rdH, rdW)
    if dt != "f64":
        # the single call (kept or recomputed logits) on the same inputs
        fb, dH2, dW2 = lce.forward_backward(c.H, c.W, c.y, c.m, chunk=max(chunk, n), z_coef=z,
                                            grad_out=g)
        check_forward(c, fb, ref)
        check_grads(c, dH2, dW2, rdH, rdW)


# ---------------------------------------------------- z-loss identities --

ZID = [
    # dtype, n, D, V, chunk, mask, z
    ("f64", 64, 64, 1000, 16, 0.25, 0.05),
    ("bf16", 300, 192, 3000, 64, 0.05, 0.05),
    ("bf16", 512, 256, 5000, 256, 0.05, 0.05),
]


@pytest.mark.parametrize("dt,n,D,V,chunk,mask,z", ZID)
def test_z_loss_identities(dt, n, D, V, chunk, mask, z):
    _say(f"case z identities {dt} n={n} D={D} V={V} z={z}")
    c0 = _case(dt, n, D, V, seed=n + 5, mask=mask, z=0.0)
    cz = _case(dt, n, D, V, seed=n + 5, mask=mask, z=z)
    f0 = c0.gpu_forward(chunk)
    fz = cz.gpu_forward(chunk)
    fs = lce.forward(c0.H, c0.W, c0.y, c0.m, chunk=chunk, z_coef=1e-4)
    # the forward never reads z_coef: identical lse and scalars, bit for bit
    assert f0.loss == fz.loss == fs.loss
    assert torch.equal(f0.lse, fz.lse) and torch.equal(f0.lse, fs.lse)
    ref0 = c0.oracle_forward(chunk)
    check_forward(c0, f0, ref0)
    dH0, dW0 = c0.gpu_backward(f0.lse, chunk)
    dHz, dWz = cz.gpu_backward(fz.lse, chunk)
    torch.cuda.synchronize()
    r0 = _oracle_grads(c0, ref0["lse"], 1.0)
    rz = _oracle_grads(cz, ref0["lse"], 1.0)
    check_grads(c0, dH0, dW0, *r0)
    check_grads(cz, dHz, dWz, *rz)
    # z on - z off = the z-only term, within the sum of the two runs' bars
    gtol = 1e-10 if dt == "f64" else 1e-2
    for name, a, b, ra, rb in (("d_hidden", dHz, dH0, rz[0], r0[0]),
                               ("d_weight", dWz, dW0, rz[1], r0[1])):
        gd = a.double().cpu().numpy() - b.double().cpu().numpy()
        rd = ra - rb
        e = float(np.max(np.abs(gd - rd))) / float(np.max(np.abs(ra)))
        _say(f"  {name}: z term max {np.max(np.abs(rd)):.3e} of {np.max(np.abs(ra)):.3e}; "
             f"difference error {e:.2e}")
        assert e <= 2 * gtol
    # vocabulary sums of d_weight: 0 without z, sum_t 2 g_z lse_t H_t with z
    m = np.ones(n) if c0.x.mask is None else c0.x.mask.astype(np.float64)
    C = m.sum()
    cs0 = dW0.double().sum(0).cpu().numpy()
    csz = dWz.double().sum(0).cpu().numpy()
    ref_cs = (m * 2.0 * (z / C) * ref0["lse"]) @ c0.H64
    scale = float(np.max(np.abs(r0[1])))
    e0 = float(np.max(np.abs(cs0))) / scale
    ez = float(np.max(np.abs(csz - ref_cs))) / scale
    _say(f"  vocabulary sum of d_weight: z off {e0:.2e}, z on vs sum_t 2 g_z lse H {ez:.2e}")
    if dt == "f64":
        assert float(np.max(np.abs(cs0))) <= 1e-9 and float(np.max(np.abs(csz - ref_cs))) <= 1e-9
    else:
        assert e0 <= 5e-2 and ez <= 5e-2
