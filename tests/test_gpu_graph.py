"""The asynchronous forward + backward, the asynchronous single call
(lce_forward_backward, with and without kept logits), a whole
vocabulary-shard step (shard forwards, asynchronous exchange, shard
backwards) and the asynchronous logits-in calls (distillation, label
cross-entropy), captured in a HIP graph
(torch.cuda.graph on the caller's stream) and replayed: every replay gives,
bit for bit, the lse, loss scalars, d_hidden and d_weight of the same calls
made eagerly, and the eager result itself matches the fp64 oracle.

The captured calls launch kernels only: no host wait, no memset node, no
allocation (every buffer, the workspace included, exists before capture).
Replays are separated by eager work on the same tensors (the outputs are
overwritten with other values), so each replay has to produce its results
afresh.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_amd import lce
from tests import synthetic as syn
from tests.test_gpu_ce import Case, check_forward, check_grads, _say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,D,V,chunk", [
    (512, 256, 12000, 128),      # several slabs, ragged last slab and token tile
    (1000, 1024, 40000, 256),    # headline d_model, packed launches
])
def test_graph_replay_matches_eager(n, D, V, chunk):
    w = syn.QWEN_BF16
    c = Case(w, n=n, D=D, V=V, seed=41)
    dev = c.H.device
    _say(f"case graph replay bf16 n={n} D={D} V={V} chunk={chunk}")
    ws = torch.empty(lce.lce_workspace_bytes(n, D, V, chunk, c.H.dtype), dtype=torch.uint8,
                     device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    dH = torch.empty_like(c.H)
    dW = torch.empty(V, D, dtype=torch.float32, device=dev)

    def step():
        st, _ = lce.lce_forward(c.H, c.W, c.y, c.m, n, D, V, chunk, c.z, lse, ws, sync=False)
        assert st == lce.OK
        st = lce.lce_backward(c.H, c.W, c.y, c.m, lse, n, D, V, chunk, c.z, 1.0, dH, dW, 0, ws)
        assert st == lce.OK

    # eager reference (also warms the planner's per-shape memo before capture)
    step()
    st, loss = lce.lce_loss_fetch(ws)
    assert st == lce.OK
    ref = (lse.clone(), dH.clone(), dW.clone(), loss.loss_sum, loss.z_sum, loss.n_counted)

    # the eager result against the oracle (sampled gradient rows)
    r = oracle.fused_forward(c.H64, c.W64, c.x.targets, mask=c.x.mask, chunk=chunk, z_coef=c.z)

    fwd = SimpleNamespace(lse=ref[0], loss=loss.as_dict())
    check_forward(c, fwd, r)
    rng = np.random.default_rng(5)
    th = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 6, replace=False)]))
    vw = np.unique(np.concatenate([[0, V - 1], rng.choice(V, 10, replace=False),
                                   c.x.targets[th]]))
    rdH = oracle.backward_dh_rows(c.H64, c.W64, c.x.targets, r["lse"], th, mask=c.x.mask,
                                  z_coef=c.z)
    rdW = oracle.backward_dw_rows(c.H64, c.W64, c.x.targets, r["lse"], vw, mask=c.x.mask,
                                  z_coef=c.z)
    check_grads(c, ref[1], ref[2], rdH, rdW, rows_h=th, rows_w=vw)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        # eager work between replays: scribble over every output
        lse.fill_(float(rep) - 7.0)
        dH.fill_(3.0)
        dW.fill_(-5.0)
        torch.cuda.synchronize()
        g.replay()
        st, loss = lce.lce_loss_fetch(ws)
        assert st == lce.OK
        _say(f"  replay {rep}: loss_sum {loss.loss_sum!r}")
        assert torch.equal(lse, ref[0])
        assert torch.equal(dH, ref[1])
        assert torch.equal(dW, ref[2])
        assert (loss.loss_sum, loss.z_sum, loss.n_counted) == ref[3:]


@pytest.mark.parametrize("n,D,V,chunk,keeps", [
    (300, 192, 3000, 300, 1),       # the logits kept: FwdKeepEpi, dlogit rows, one backward launch
    (512, 256, 12000, 128, 0),      # chunk below the batch: the two-call algorithm inside
])
def test_graph_replay_single_call(n, D, V, chunk, keeps):
    """lce_forward_backward without a host result (asynchronous) captured and
    replayed: every replay equals the eager call bit for bit."""
    w = syn.QWEN_BF16
    c = Case(w, n=n, D=D, V=V, seed=43)
    dev = c.H.device
    _say(f"case graph replay single call bf16 n={n} D={D} V={V} chunk={chunk}")
    assert lce.lce_forward_backward_keeps_logits(n, D, V, chunk, c.H.dtype) == keeps
    nbytes = lce.lce_forward_backward_workspace_bytes(n, D, V, chunk, c.H.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    dH = torch.empty_like(c.H)
    dW = torch.empty(V, D, dtype=torch.float32, device=dev)

    def step():
        st, _ = lce.lce_forward_backward(c.H, c.W, c.y, c.m, n, D, V, chunk, c.z, 1.0, lse, dH,
                                         dW, 0, ws, sync=False)
        assert st == lce.OK

    step()
    st, loss = lce.lce_loss_fetch(ws)
    assert st == lce.OK
    ref = (lse.clone(), dH.clone(), dW.clone(), loss.loss_sum, loss.z_sum, loss.n_counted)
    r = oracle.fused_forward(c.H64, c.W64, c.x.targets, mask=c.x.mask, chunk=chunk, z_coef=c.z)
    check_forward(c, SimpleNamespace(lse=ref[0], loss=loss.as_dict()), r)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        lse.fill_(float(rep) + 11.0)
        dH.fill_(-2.0)
        dW.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        st, loss = lce.lce_loss_fetch(ws)
        assert st == lce.OK
        _say(f"  replay {rep}: loss_sum {loss.loss_sum!r}")
        assert torch.equal(lse, ref[0])
        assert torch.equal(dH, ref[1])
        assert torch.equal(dW, ref[2])
        assert (loss.loss_sum, loss.z_sum, loss.n_counted) == ref[3:]


def test_graph_replay_shard_step():
    """A whole vocabulary-shard step -- every shard's forward, the asynchronous
    exchange, every shard's backward with the d_hidden partials added up --
    captured and replayed: every replay equals the eager step bit for bit, and
    the eager loss matches the oracle's."""
    w = syn.QWEN_BF16
    n, D, V, chunk = 300, 128, 3000, 64
    bounds = [0, 1024, 1100, 3000]
    c = Case(w, n=n, D=D, V=V, seed=47)
    dev = c.H.device
    _say(f"case graph replay shard step bf16 n={n} D={D} V={V} bounds={bounds}")
    P = len(bounds) - 1
    rows = max(bounds[q + 1] - bounds[q] for q in range(P))
    ws = torch.empty(lce.lce_workspace_bytes(n, D, rows, chunk, c.H.dtype), dtype=torch.uint8,
                     device=dev)
    mws = torch.empty(lce.lce_distill_workspace_bytes(n, 1), dtype=torch.uint8, device=dev)
    stats = torch.empty(P, 3, n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    part = torch.empty(n, D, dtype=torch.float32, device=dev)
    dH = torch.empty(n, D, dtype=torch.float32, device=dev)
    dW = torch.empty(V, D, dtype=torch.float32, device=dev)

    def step():
        for q in range(P):
            a, b = bounds[q], bounds[q + 1]
            st = lce.lce_shard_forward(c.H, c.W[a:b], c.y, n, D, b - a, a, V, chunk, stats[q],
                                       ws)
            assert st == lce.OK
        st, _ = lce.lce_shard_merge(stats, P, c.m, n, lse, mws, sync=False)
        assert st == lce.OK
        for q in range(P):
            a, b = bounds[q], bounds[q + 1]
            st = lce.lce_shard_backward(c.H, c.W[a:b], c.y, c.m, lse, n, D, b - a, a, V, chunk,
                                        c.z, 1.0, part, dW[a:b], 0, ws)
            assert st == lce.OK
            if q == 0:
                dH.copy_(part)
            else:
                dH.add_(part)

    step()
    assert lce.lce_loss_fetch(ws)[0] == lce.OK       # the shard calls' target guards
    st, loss = lce.lce_loss_fetch(mws)
    assert st == lce.OK
    ref = (lse.clone(), dH.clone(), dW.clone(), loss.loss_sum, loss.z_sum, loss.n_counted)
    r = oracle.fused_forward(c.H64, c.W64, c.x.targets, mask=c.x.mask, chunk=chunk, z_coef=c.z)
    check_forward(c, SimpleNamespace(lse=ref[0], loss=loss.as_dict()), r)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        stats.fill_(5.0)
        lse.fill_(float(rep) - 1.0)
        dH.fill_(9.0)
        dW.fill_(-4.0)
        torch.cuda.synchronize()
        g.replay()
        assert lce.lce_loss_fetch(ws)[0] == lce.OK
        st, loss = lce.lce_loss_fetch(mws)
        assert st == lce.OK
        _say(f"  replay {rep}: loss_sum {loss.loss_sum!r}")
        assert torch.equal(lse, ref[0])
        assert torch.equal(dH, ref[1])
        assert torch.equal(dW, ref[2])
        assert (loss.loss_sum, loss.z_sum, loss.n_counted) == ref[3:]


def test_graph_replay_logits_in_calls():
    """The asynchronous distillation call (the three objectives) and label
    cross-entropy from logits captured in one graph: every replay equals the
    eager calls bit for bit (gradients and the scalars lce_loss_fetch reads)."""
    dev = torch.device("cuda:0")
    n, V = 37, 3000
    _say(f"case graph replay logits-in calls bf16 n={n} V={V}")
    d = syn.distill_inputs(syn.DISTILL_BF16, n_tok=n, vocab=V, seed=53, dtype="bf16")
    S, U = d.student.to(dev), d.teacher.to(dev)
    m = torch.from_numpy(d.mask).to(dev)
    y = torch.from_numpy(syn.label_inputs(syn.LABEL_BF16, n_tok=n, vocab=V, seed=54).targets).to(dev)
    nb = lce.lce_distill_workspace_bytes(n, V)
    wss = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(4)]
    gs = [torch.empty_like(S) for _ in range(4)]

    def step():
        for obj in range(3):
            st, _ = lce.lce_distill_fwd_bwd(S, U, m, n, V, obj, 2.0, 1e-3, 1.1, gs[obj], wss[obj],
                                            sync=False)
            assert st == lce.OK
        st, _ = lce.lce_ce_logits_fwd_bwd(S, y, m, n, V, 1e-3, 0.9, gs[3], wss[3], sync=False)
        assert st == lce.OK

    def fetch_all():
        res = []
        for ws in wss:
            st, loss = lce.lce_loss_fetch(ws)
            assert st == lce.OK
            res.append((loss.loss_sum, loss.z_sum, loss.n_counted))
        return res

    step()
    ref_g = [g.clone() for g in gs]
    ref_l = fetch_all()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        for g in gs:
            g.fill_(float(rep) + 2.0)
        torch.cuda.synchronize()
        gr.replay()
        assert fetch_all() == ref_l
        for g, r in zip(gs, ref_g):
            assert torch.equal(g, r)
