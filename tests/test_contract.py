"""Host-side contract of liblce.so (no GPU): the library loads, exports every
function include/lce.h declares, and its integer contract equals the
independent oracle's bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_amd import lce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "lce.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lce_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"lce_dims_check", "lce_chunk_check", "lce_peak_cells", "lce_forward",
            "lce_backward", "lce_distill_fwd_bwd"} <= set(names)
    L = ctypes.CDLL(lce.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_printed_values_through_the_library():
    r = lce.lce_peak_cells(2048, 151936, 256)
    assert r == {"chunked_cells": 38895616.0, "materialized_cells": 311164928.0, "ratio": 8.0,
                 "n_chunks": 8, "status": 580}
    assert lce.lce_dims_check(2048, 4096, 151936) == 580
    assert lce.lce_chunk_check(2048, 151936) == 587
    assert lce.lce_chunk_check(256, 151936) == 580
    assert lce.lce_chunk_check(1024, 151936) == 587   # the swept chunk 1024 is refused


def test_contract_matches_oracle_on_a_sweep():
    rng = np.random.default_rng(3)
    vals = [0, 1, 2, 3, 7, 255, 256, 883, 884, 1024, 2 ** 10, 2 ** 16, 2 ** 16 + 1, 2 ** 17,
            2 ** 24, 2 ** 24 + 1, 2 ** 27, 2 ** 27 + 1, 2 ** 40, -1, -(2 ** 40)]
    vals += [int(x) for x in rng.integers(1, 2 ** 31, 40)]
    for a in vals:
        for b in vals:
            assert lce.lce_chunk_check(a, b) == oracle.chunk_check(a, b), (a, b)
            assert lce.lce_logit_cells(a, b) == oracle.logit_cells(a, b), (a, b)
    trip = [(int(a), int(b), int(c)) for a, b, c in rng.choice(vals, size=(2000, 3))]
    trip += [(2 ** 24, 2 ** 16, 64), (2 ** 24, 2 ** 16, 65), (2048, 1024, 151936)]
    for n, d, v in trip:
        assert lce.lce_dims_check(n, d, v) == oracle.dims_check(n, d, v), (n, d, v)
        assert lce.lce_work_fits(n, d, v, 2 ** 46) == oracle.work_fits(n, d, v, 2 ** 46)
        assert lce.lce_peak_cells(n, v, d) == oracle.peak_cells(n, v, d), (n, v, d)


def test_status_names_match_oracle():
    for code in list(range(570, 600)) + [-1, 0, 600, 2 ** 31 - 1]:
        assert lce.lce_status_name(code) == oracle.status_name(code), code


def test_workspace_sizes():
    for dt in (lce.BF16, lce.F64):
        b = lce.lce_workspace_bytes(2048, 1024, 151936, 256, dt)
        assert b > 0
        # the logit-gradient slab never exceeds chunk*vocab cells
        assert b < 256 * 151936 * (2 if dt == lce.BF16 else 8) + 2048 * 1024 * 16 * 8 + 2 ** 24
    assert lce.lce_workspace_bytes(2048, 1024, 151936, 1024, lce.BF16) == -587
    assert lce.lce_workspace_bytes(0, 1024, 151936, 256, lce.BF16) == -581
    assert lce.lce_workspace_bytes(64, 64, 1000, 16, lce.F32) == -590
    assert lce.lce_distill_workspace_bytes(4096, 151936) > 0
    assert lce.lce_distill_workspace_bytes(0, 5) == -581


@pytest.mark.parametrize("n,D,V,chunk", [(64, 64, 1000, 16), (2048, 1024, 151936, 256),
                                         (8192, 4096, 128256, 512), (7, 3, 5, 1),
                                         (2048, 1024, 151936, 1), (100000, 64, 5000, 3)])
def test_workspace_monotone_and_bounded(n, D, V, chunk):
    for dt in (lce.BF16, lce.F64):
        b = lce.lce_workspace_bytes(n, D, V, chunk, dt)
        assert b > 0


def test_single_call_workspace():
    """lce_forward_backward keeps the batch's logits only when a 16-bit batch
    fits one chunk; the kept logits take at most chunk*vocab fp32 cells."""
    f = lce.lce_forward_backward_workspace_bytes
    # the headline (chunk 256 < 2048 tokens): the two-call workspace
    for dt in (lce.BF16, lce.F16, lce.F64):
        assert f(2048, 1024, 151936, 256, dt) == lce.lce_workspace_bytes(2048, 1024, 151936, 256,
                                                                          dt)
    # fp64 never keeps logits
    assert f(512, 1024, 151936, 512, lce.F64) == lce.lce_workspace_bytes(512, 1024, 151936, 512,
                                                                          lce.F64)
    for n, D, V, chunk in [(512, 4096, 151936, 512), (256, 1024, 151936, 256),
                           (300, 192, 3000, 300), (1, 64, 33, 32), (517, 256, 2100, 600)]:
        single, two = f(n, D, V, chunk, lce.BF16), lce.lce_workspace_bytes(n, D, V, chunk,
                                                                           lce.BF16)
        assert single > two
        sp = 64
        extra = 4 * V * chunk + 4 * sp * n * D + 2 * D * (n + 63) // 64 * 64 + 8 * n + 5 * 256
        assert single <= two + extra
    # a batch one row larger than the chunk goes the two-call way
    assert f(301, 192, 3000, 300, lce.BF16) == lce.lce_workspace_bytes(301, 192, 3000, 300,
                                                                        lce.BF16)
    assert f(2048, 1024, 151936, 1024, lce.BF16) == -587
    assert f(0, 1024, 151936, 256, lce.BF16) == -581
    assert f(64, 64, 1000, 64, lce.F32) == -590


def test_single_call_dispatch():
    """lce_forward_backward_keeps_logits: the launch-cost model keeps the
    logits where that measured faster (512 x 4096, 512 x 1024 and 256 x 1024
    heads of 151936 rows) and takes the two-call algorithm where the model
    puts keeping behind (768 x 512: the recompute saved is small against the
    kept logits' traffic); the workspace follows the choice."""
    k = lce.lce_forward_backward_keeps_logits
    f = lce.lce_forward_backward_workspace_bytes
    w = lce.lce_workspace_bytes
    assert k(512, 4096, 151936, 512, lce.BF16) == 1
    assert k(256, 1024, 151936, 256, lce.BF16) == 1
    assert k(512, 1024, 151936, 512, lce.BF16) == 1
    assert k(768, 512, 151936, 768, lce.BF16) == 0
    assert f(768, 512, 151936, 768, lce.BF16) == w(768, 512, 151936, 768, lce.BF16)
    assert k(512, 4096, 151936, 512, lce.F16) == 1
    assert k(512, 4096, 151936, 512, lce.F64) == 0        # fp64 never keeps
    assert k(2048, 1024, 151936, 256, lce.BF16) == 0      # the batch exceeds the chunk
    assert k(96, 100, 777, 96, lce.BF16) == 0             # d_model not a multiple of 64
    assert k(2048, 1024, 151936, 1024, lce.BF16) == -587
    assert k(0, 1024, 151936, 256, lce.BF16) == -581
    assert k(64, 64, 1000, 64, lce.F32) == -590
    for n, D, V, chunk in [(300, 192, 3000, 300), (200, 128, 3000, 256), (130, 128, 2000, 132)]:
        assert k(n, D, V, chunk, lce.BF16) == 1, (n, D, V)
        assert f(n, D, V, chunk, lce.BF16) > w(n, D, V, chunk, lce.BF16)


def test_loss_fetch_refuses_short_workspace_without_device():
    ws = torch.zeros(100, dtype=torch.uint8)
    assert lce.lce_loss_fetch(ws, stream=0)[0] == 582
    assert lce.lce_loss_fetch(torch.zeros(1024, dtype=torch.int32), stream=0)[0] == 590


def test_ce_logits_refusals_without_device():
    """Host-side validation of lce_ce_logits_fwd_bwd returns before any
    device call (dims, scalars, dtypes, lengths in that order)."""
    Z = torch.zeros(4, 16, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    ws = torch.zeros(lce.lce_distill_workspace_bytes(4, 16) + 256, dtype=torch.uint8)
    call = lambda **kw: lce.lce_ce_logits_fwd_bwd(**{**dict(
        logits=Z, targets=y, loss_mask=None, n_tok=4, vocab=16, z_coef=0.0, grad_out=1.0,
        grad_logits=Z, workspace=ws, stream=0), **kw})[0]
    assert call(n_tok=0) == 581
    assert call(vocab=0) == 581
    assert call(z_coef=float("inf")) == 585
    assert call(grad_out=float("nan")) == 585
    assert call(targets=y.int()) == 590
    assert call(grad_logits=Z.float()) == 590
    assert call(loss_mask=torch.zeros(4, dtype=torch.int32)) == 590
    assert call(logits=Z[:3]) == 582
    assert call(targets=y[:3]) == 582
    assert call(workspace=ws[:16]) == 582
