"""GPU parity of the vocabulary-shard path (lce_shard_forward / lce_shard_merge
/ lce_shard_backward) against the CPU fp64 oracle of the whole head, through
the C ABI: the shards' exchange must reproduce the unsharded loss, lse and
gradients.  Tolerances as the unsharded path (fp64: 1e-10; bf16: loss and lse
2e-3 relative, gradients 1e-2 * max|ref|)."""
import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_amd import lce
from tests import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = {"f64": (1e-10, 1e-10), "bf16": (2e-3, 1e-2)}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def normwise(a, ref):
    return float(np.max(np.abs(a - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def run_shards(H, W, y, m, bounds, chunk, z, grad_out=1.0, backward=True):
    """Every shard's forward, the exchange, every shard's backward.  Returns
    (loss, lse, stats [P][3][n], d_hidden = sum of partials, d_weight)."""
    dev = H.device
    n, D = H.shape
    V = W.shape[0]
    acc = torch.float64 if H.dtype == torch.float64 else torch.float32
    P = len(bounds) - 1
    stats = torch.empty(P, 3, n, dtype=acc, device=dev)
    wss = []
    for q in range(P):
        a, b = bounds[q], bounds[q + 1]
        ws = lce.workspace_for(n, D, b - a, chunk, H.dtype, dev)
        st = lce.lce_shard_forward(H, W[a:b], y, n, D, b - a, a, V, chunk, stats[q], ws)
        assert st == 580, (q, st)
        wss.append(ws)
    lse = torch.empty(n, dtype=acc, device=dev)
    mws = torch.empty(lce.lce_distill_workspace_bytes(n, 1), dtype=torch.uint8, device=dev)
    st, out = lce.lce_shard_merge(stats, P, m, n, lse, mws)
    assert st == 580
    if not backward:
        return out.as_dict(), lse, stats, None, None
    dH = torch.zeros(n, D, dtype=torch.float64, device=dev)
    dW = torch.empty(V, D, dtype=acc, device=dev)
    part = torch.empty(n, D, dtype=acc, device=dev)
    for q in range(P):
        a, b = bounds[q], bounds[q + 1]
        st = lce.lce_shard_backward(H, W[a:b], y, m, lse, n, D, b - a, a, V, chunk, z, grad_out,
                                    part, dW[a:b], 0, wss[q])
        assert st == 580, (q, st)
        dH += part.double()          # the exchange of the d_hidden partials
    return out.as_dict(), lse, stats, dH, dW


SHARDS = [
    # dtype, n, D, V, bounds, chunk, mask, z
    ("f64", 70, 64, 1000, [0, 300, 301, 1000], 16, 0.2, 1e-3),
    ("f64", 33, 37, 500, [0, 250, 500], 7, None, 0.0),
    ("bf16", 300, 128, 3000, [0, 1024, 1100, 3000], 64, 0.05, 1e-4),
    ("bf16", 130, 96, 2000, [0, 500, 1999, 2000], 130, None, 1e-3),   # one-row shard
    ("bf16", 257, 256, 5000, [0, 1280, 2560, 3840, 5000], 256, 0.1, 1e-4),
]


@pytest.mark.parametrize("dt,n,D,V,bounds,chunk,mask,z", SHARDS)
def test_shards_match_the_whole_head(dt, n, D, V, bounds, chunk, mask, z):
    _say(f"case shards {dt} n={n} D={D} V={V} bounds={bounds} chunk={chunk}")
    dev = _dev()
    w = syn.TINY_F64 if dt == "f64" else syn.QWEN_BF16
    x = syn.ce_inputs(w, n_tok=n, d_model=D, vocab=V, seed=n + V)
    if mask is not None:
        x.mask = syn.exact_mask(np.random.default_rng(77 + n), n, mask)
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    m = torch.from_numpy(x.mask).to(dev) if x.mask is not None else None
    out, lse, stats, dH, dW = run_shards(H, W, y, m, bounds, chunk, z, grad_out=1.25)
    H64, W64 = x.hidden64(), x.weight64()
    ref = oracle.fused_forward(H64, W64, x.targets, mask=x.mask, chunk=chunk, z_coef=z)
    lt, gt = TOL[dt]
    assert out["n_counted"] == ref["n_counted"]
    el = abs(out["loss_mean"] - ref["loss_mean"]) / abs(ref["loss_mean"])
    ez = abs(out["z_mean"] - ref["z_mean"]) / abs(ref["z_mean"])
    ell = normwise(lse.double().cpu().numpy(), ref["lse"])
    _say(f"  loss rel {el:.2e} z rel {ez:.2e} lse {ell:.2e}")
    assert el <= lt and ez <= lt and ell <= lt
    # every shard's record against the oracle on that shard's rows alone
    st = stats.double().cpu().numpy()
    for q in range(len(bounds) - 1):
        a, b = bounds[q], bounds[q + 1]
        own = (x.targets >= a) & (x.targets < b)
        yl = np.where(own, x.targets - a, 0)
        r = oracle.fused_forward(H64, W64[a:b], yl, chunk=1, z_coef=0.0)
        lse_q = st[q, 0] + np.log(st[q, 1])
        assert normwise(lse_q, r["lse"]) <= lt, q
        zq = r["lse"] - r["loss_tok"]                    # z[t][y_t] on the shard
        assert normwise(st[q, 2][own], zq[own]) <= lt if own.any() else True
        assert np.all(st[q, 2][~own] == 0.0)
    rdH, rdW = oracle.backward(H64, W64, x.targets, ref["lse"], mask=x.mask, z_coef=z,
                               grad_out=1.25)
    eh = normwise(dH.cpu().numpy(), rdH)
    ew = normwise(dW.double().cpu().numpy(), rdW)
    _say(f"  dH {eh:.2e} dW {ew:.2e}")
    assert eh <= gt and ew <= gt


def test_f16_shards():
    """fp16 inputs in three shards; grad_out carries an fp16 loss scale."""
    import dataclasses
    dev = _dev()
    w = dataclasses.replace(syn.QWEN_BF16, dtype="f16")
    n, D, V, chunk, z, go = 300, 128, 3000, 64, 1e-4, 1024.0
    x = syn.ce_inputs(w, n_tok=n, d_model=D, vocab=V, seed=71)
    x.mask = syn.exact_mask(np.random.default_rng(71), n, 0.05)
    H, W = x.hidden.to(dev), x.weight.to(dev)
    assert H.dtype == torch.float16
    y = torch.from_numpy(x.targets).to(dev)
    m = torch.from_numpy(x.mask).to(dev)
    out, lse, _, dH, dW = run_shards(H, W, y, m, [0, 1024, 2048, 3000], chunk, z, grad_out=go)
    H64, W64 = x.hidden64(), x.weight64()
    ref = oracle.fused_forward(H64, W64, x.targets, mask=x.mask, chunk=chunk, z_coef=z)
    el = abs(out["loss_mean"] - ref["loss_mean"]) / abs(ref["loss_mean"])
    rdH, rdW = oracle.backward(H64, W64, x.targets, ref["lse"], mask=x.mask, z_coef=z,
                               grad_out=go)
    eh = normwise(dH.cpu().numpy(), rdH)
    ew = normwise(dW.double().cpu().numpy(), rdW)
    _say(f"  f16 shards: loss rel {el:.2e} dH {eh:.2e} dW {ew:.2e}")
    assert el <= 2e-3 and eh <= 1e-2 and ew <= 1e-2


@pytest.mark.parametrize("dt", ["bf16", "f64"])
def test_async_merge_matches_the_synchronous_merge(dt):
    """lce_shard_merge without a host result returns once enqueued; the lse it
    writes and the scalars lce_loss_fetch then returns equal the synchronous
    call's bit for bit."""
    w = syn.QWEN_BF16 if dt == "bf16" else syn.TINY_F64
    x = syn.ce_inputs(w, n_tok=200, d_model=64, vocab=3000, seed=17)
    dev = _dev()
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    mask = syn.exact_mask(np.random.default_rng(3), 200, 0.1)
    m = torch.from_numpy(mask).to(dev)
    _say(f"case async shard merge {dt} n=200 V=3000 in 3 shards")
    ref, lse, stats, _, _ = run_shards(H, W, y, m, [0, 1000, 2048, 3000], 64, 1e-3,
                                      backward=False)
    lse2 = torch.full_like(lse, -3.0)
    mws = torch.empty(lce.lce_distill_workspace_bytes(200, 1), dtype=torch.uint8, device=dev)
    st, out = lce.lce_shard_merge(stats, 3, m, 200, lse2, mws, sync=False)
    assert st == 580 and out is None
    st, loss = lce.lce_loss_fetch(mws)
    assert st == 580
    assert torch.equal(lse2, lse)
    assert loss.as_dict() == ref
    # refusals come back before anything is enqueued, with or without a result
    assert lce.lce_shard_merge(stats, 0, None, 200, lse2, mws, sync=False)[0] == 581
    assert lce.lce_shard_merge(stats, 4, None, 200, lse2, mws, sync=False)[0] == 582


@pytest.mark.parametrize("dt", ["bf16", "f64"])
def test_one_shard_is_the_unsharded_call(dt):
    """A single shard over the whole head runs the same kernels: lse, loss,
    d_weight and the rounded d_hidden are identical bit for bit."""
    dev = _dev()
    w = syn.TINY_F64 if dt == "f64" else syn.QWEN_BF16
    n, D, V, chunk = (90, 64, 900, 30) if dt == "f64" else (200, 128, 3000, 100)
    x = syn.ce_inputs(w, n_tok=n, d_model=D, vocab=V, seed=3)
    x.mask = syn.exact_mask(np.random.default_rng(3), n, 0.1)
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    m = torch.from_numpy(x.mask).to(dev)
    out, lse, _, dH, dW = run_shards(H, W, y, m, [0, V], chunk, 1e-3)
    f = lce.forward(H, W, y, m, chunk=chunk, z_coef=1e-3)
    dh1, dw1 = lce.backward(H, W, y, f.lse, m, chunk=chunk, z_coef=1e-3)
    assert out["loss_sum"] == f.loss["loss_sum"] and out["z_sum"] == f.loss["z_sum"]
    assert torch.equal(lse, f.lse)
    assert torch.equal(dW, dw1)
    assert torch.equal(dH.to(H.dtype), dh1)


def test_shard_refusals():
    dev = _dev()
    x = syn.ce_inputs(syn.QWEN_BF16, n_tok=16, d_model=64, vocab=300, seed=5)
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    stats = torch.full((3, 16), 7.0, dtype=torch.float32, device=dev)
    ws = lce.workspace_for(16, 64, 100, 16, torch.bfloat16, dev)
    call = lambda **kw: lce.lce_shard_forward(**{**dict(
        hidden=H, weight_shard=W[100:200], targets=y, n_tok=16, d_model=64, vocab_shard=100,
        vocab_offset=100, vocab_total=300, chunk=16, stats=stats, workspace=ws), **kw})
    assert call(vocab_offset=201) == 582          # rows past the head
    assert call(vocab_offset=-1) == 582
    assert call(vocab_total=-5) == 581
    assert call(stats=stats.double()) == 590
    assert call(stats=stats[0]) == 582
    bad = y.clone()
    bad[3] = 300                                  # outside the whole head
    assert call(targets=bad) == 580               # enqueued; the guard's verdict is fetched
    assert lce.lce_loss_fetch(ws)[0] == 586
    torch.cuda.synchronize()
    assert torch.all(stats == 7.0)
    assert call() == 580
    assert lce.lce_loss_fetch(ws)[0] == 580
    lse = torch.empty(16, dtype=torch.float32, device=dev)
    mws = torch.empty(lce.lce_distill_workspace_bytes(16, 1), dtype=torch.uint8, device=dev)
    assert lce.lce_shard_merge(stats, 0, None, 16, lse, mws)[0] == 581
    assert lce.lce_shard_merge(stats, 2, None, 16, lse, mws)[0] == 582   # one record only
    assert lce.lce_shard_merge(stats, 1, None, 16, lse.double(), mws)[0] == 590


def test_shards_of_the_headline_head():
    """2048 x 1024 x 151936 bf16 (chunk 256, z 1e-4, 5% masked) in four shards
    of 37984 rows: the lse and d_hidden of sampled tokens match the oracle
    (d_hidden of a token needs only that token's lse); the loss and d_weight
    equal the unsharded call's (itself checked against the oracle at this
    size) to rounding."""
    w = syn.QWEN_BF16
    dev = _dev()
    _say(f"case {w.name} in 4 shards: generating inputs")
    x = syn.ce_inputs(w)
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    m = torch.from_numpy(x.mask).to(dev)
    V = w.vocab
    bounds = [0, V // 4, V // 2, 3 * V // 4, V]
    out, lse, _, dH, dW = run_shards(H, W, y, m, bounds, w.chunk, w.z_coef)
    f = lce.forward(H, W, y, m, chunk=w.chunk, z_coef=w.z_coef)
    _, dw1 = lce.backward(H, W, y, f.lse, m, chunk=w.chunk, z_coef=w.z_coef)
    el = abs(out["loss_mean"] - f.loss["loss_mean"]) / f.loss["loss_mean"]
    ew = normwise(dW.double().cpu().numpy(), dw1.double().cpu().numpy())
    _say(f"  merged loss {out['loss_mean']:.9g} unsharded {f.loss['loss_mean']:.9g} rel {el:.2e}"
         f"; d_weight vs unsharded {ew:.2e}")
    assert el <= 1e-6 and out["n_counted"] == f.loss["n_counted"] and ew <= 1e-3
    rng = np.random.default_rng(41)
    th = np.sort(rng.choice(w.n_tok, 5, replace=False))
    H64, W64 = x.hidden64(), x.weight64()
    _say(f"  oracle on tokens {th.tolist()}")
    ref = oracle.fused_forward(H64[th], W64, x.targets[th], chunk=1)
    assert normwise(lse[torch.from_numpy(th).to(dev)].double().cpu().numpy(), ref["lse"]) <= 2e-3
    lse_in = np.zeros(w.n_tok)
    lse_in[th] = ref["lse"]          # the oracle's lse of the sampled tokens
    rdH = oracle.backward_dh_rows(H64, W64, x.targets, lse_in, th, mask=x.mask, z_coef=w.z_coef)
    eh = normwise(dH.cpu().numpy()[th], rdH)
    _say(f"  sampled dH {eh:.2e}")
    assert eh <= 1e-2
