"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

Default workload: the Qwen3-0.6B-shaped LM head, 2048 tokens x d_model 1024 x
vocab 151936, bf16 inputs with fp32 accumulation, chunk 256, z-loss 1e-4, 5%
of tokens masked, synthetic seeded inputs already resident in HBM.  One step
= lce_forward + lce_backward as a training loop makes them; neither call waits
for the device, and the loss scalars and the target guard's verdict are read
back once after the timed steps (lce_loss_fetch).  Prints one JSON line.

Timing: the K timed steps run with nothing recorded between kernels (value,
ms_per_step, from the host clock around the K steps and a final sync); a
per-step pass records an event between consecutive steps (step_ms_median,
step_ms_min).  A third pass repeats the K steps with HIP events that the
library records around every kernel launch on the launch stream
(lce_forward_timed / lce_backward_timed); those give the per-kind kernel
durations and roofline.achieved.  Events add idle time between kernels, so
that pass never feeds the step time.

Side records (default run): fp16 inputs, the single call, vocabulary shards,
the fp64 chunk sweep (128/256/512, and 1024 refused with 587), the
8192 x 4096 x 128256 head, distillation and label CE throughput, and a
practical MFMA ceiling (hipBLASLt on 8192^3 with the sampled clock).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F64_TFLOPS = 78.6         # MI355X fp64 MFMA
PEAK_HBM_GBS = 8000.0

GEMM_KINDS = ["fwd_gemm", "dlogit_gemm", "dw_gemm", "dh_gemm", "bwd_gemm"]
# GEMM passes (2*n*D*V flops each) one step's launches of a kind perform
GEMM_PASSES = {"fwd_gemm": 1, "dlogit_gemm": 1, "dw_gemm": 1, "dh_gemm": 1, "bwd_gemm": 3}
ALL_KINDS = ["guard", "fwd_gemm", "fwd_merge", "reduce", "dlogit_gemm", "dw_gemm", "dh_gemm",
             "dh_final", "bwd_gemm"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_sha256() -> str:
    """Digest of the HIP sources the GEMM kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "lm_head_linear_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profiles(workload: str, kind: str):
    """HBM bytes per launch of `kind` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a known-size copy), or None when
    there is none for this workload or the kernel sources changed since."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.md"))):
        for line in open(path):
            if not line.startswith("traffic: "):
                continue
            rec = json.loads(line[len("traffic: "):])
            if rec.get("workload") != workload:
                continue
            if rec.get("sources_sha256") != kernel_sources_sha256():
                return None
            v = rec.get("per_launch_bytes", {}).get(kind)
            return None if v is None else int(v)
    return None


def distill_measure(lce, torch, np, dev, steps: int):
    """lce_distill_fwd_bwd on the 4096 x 151936 bf16 distillation workload
    (T = 2, 10% masked, z 1e-4) for the three objectives: kernel time from
    HIP events and HBM throughput on the algorithmic bytes 2*V*(2*C + n) + n
    (student and teacher read for counted rows, the gradient written for every
    row, the mask read)."""
    from tests import synthetic as syn
    w = syn.DISTILL_BF16
    log(f"bench: distillation {w.name}: generating inputs")
    x = syn.distill_inputs(w)
    S, U = x.student.to(dev), x.teacher.to(dev)
    mk = torch.from_numpy(x.mask).to(dev)
    n, V = S.shape
    C = int(x.mask.sum())
    g = torch.empty_like(S)
    ws = torch.empty(lce.lce_distill_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
    nbytes = 2 * V * (2 * C + n) + n
    res = {"workload": w.name, "n_tok": n, "vocab": V, "counted": C, "temperature": w.temperature,
           "algorithmic_bytes": nbytes, "peak_GBs": PEAK_HBM_GBS, "objectives": {}}
    for obj, name in ((0, "ce"), (1, "forward_kl"), (2, "reverse_kl")):
        def call(timer=None):
            st, out = lce.lce_distill_fwd_bwd(S, U, mk, n, V, obj, w.temperature, w.z_coef, 1.0, g,
                                             ws, timer=timer)
            if st != lce.OK:
                raise lce.LceError(st, "lce_distill_fwd_bwd")
            return out
        for _ in range(2):
            call()
        t0 = time.perf_counter()
        for _ in range(steps):
            out = call()
        wall = (time.perf_counter() - t0) / steps * 1e3
        timer = lce.KernelTimer(["distill"], capacity=steps * 4)
        for _ in range(steps):
            call(timer)
        torch.cuda.synchronize()
        d = timer.durations_ms("distill")
        k_ms = float(np.sum(d)) / steps
        res["objectives"][name] = {"call_ms": round(wall, 4), "kernel_ms": round(k_ms, 4),
                                   "GBs": round(nbytes / (k_ms / 1e3) / 1e9, 1),
                                   "frac": round(nbytes / (k_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                                   "loss": out.loss_mean}
    return res


def label_measure(lce, torch, np, dev, steps: int):
    """lce_ce_logits_fwd_bwd on 4096 x 151936 bf16 logits (10% masked, z
    1e-4), with the gradient and loss only: kernel time from HIP events and
    HBM throughput on the algorithmic bytes (logits read once for counted
    rows, the gradient written for every row, targets and mask read)."""
    from tests import synthetic as syn
    w = syn.LABEL_BF16
    log(f"bench: label cross-entropy {w.name}: generating inputs")
    x = syn.label_inputs(w)
    Z = x.logits.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    mk = torch.from_numpy(x.mask).to(dev)
    n, V = Z.shape
    C = int(x.mask.sum())
    g = torch.empty_like(Z)
    ws = torch.empty(lce.lce_distill_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
    res = {"workload": w.name, "n_tok": n, "vocab": V, "counted": C, "peak_GBs": PEAK_HBM_GBS,
           "modes": {}}
    for mode, grad, nbytes in (("fwd_bwd", g, 2 * V * (C + n) + 9 * n),
                               ("loss_only", None, 2 * V * C + 9 * n)):
        def call(timer=None):
            st, out = lce.lce_ce_logits_fwd_bwd(Z, y, mk, n, V, w.z_coef, 1.0, grad, ws,
                                                timer=timer)
            if st != lce.OK:
                raise lce.LceError(st, "lce_ce_logits_fwd_bwd")
            return out
        for _ in range(2):
            call()
        t0 = time.perf_counter()
        for _ in range(steps):
            out = call()
        wall = (time.perf_counter() - t0) / steps * 1e3
        timer = lce.KernelTimer(["label_ce"], capacity=steps * 4)
        for _ in range(steps):
            call(timer)
        torch.cuda.synchronize()
        k_ms = float(np.sum(timer.durations_ms("label_ce"))) / steps
        res["modes"][mode] = {"algorithmic_bytes": nbytes, "call_ms": round(wall, 4),
                              "kernel_ms": round(k_ms, 4),
                              "GBs": round(nbytes / (k_ms / 1e3) / 1e9, 1),
                              "frac": round(nbytes / (k_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                              "loss": out.loss_mean}
    return res


def shard_measure(lce, torch, np, dev, w, H, W, y, m, steps: int, shards: int):
    """The same training step as vocabulary shards run one after another on
    this GPU (each shard's forward, the exchange, each shard's backward with
    its d_hidden partial added up, no host wait inside the step): what one
    GPU's share of a vocab-parallel head costs, and the exchange's overhead
    against the unsharded step.  Each shard call gets chunk = the unsharded
    chunk x shards, so that a shard holds as many logit cells (chunk x its
    rows) as the unsharded call does (chunk x vocab): the peak logit memory
    of one GPU of a vocab-parallel head at the unsharded call's budget."""
    n, D = H.shape
    V = W.shape[0]
    chunk = w.chunk * shards
    bounds = [V * q // shards // 256 * 256 for q in range(shards)] + [V]
    acc = torch.float64 if H.dtype == torch.float64 else torch.float32
    stats = torch.empty(shards, 3, n, dtype=acc, device=dev)
    lse = torch.empty(n, dtype=acc, device=dev)
    part = torch.empty(n, D, dtype=acc, device=dev)
    dH = torch.empty(n, D, dtype=acc, device=dev)
    dW = torch.empty(V, D, dtype=acc, device=dev)
    rows = max(bounds[q + 1] - bounds[q] for q in range(shards))
    ws = torch.empty(lce.lce_workspace_bytes(n, D, rows, chunk, H.dtype), dtype=torch.uint8,
                     device=dev)
    mws = torch.empty(lce.lce_distill_workspace_bytes(n, 1), dtype=torch.uint8, device=dev)

    def step():
        for q in range(shards):
            a, b = bounds[q], bounds[q + 1]
            st = lce.lce_shard_forward(H, W[a:b], y, n, D, b - a, a, V, chunk, stats[q], ws)
            if st != lce.OK:
                raise lce.LceError(st, "lce_shard_forward")
        # asynchronous exchange: no host wait anywhere in the step
        st, _ = lce.lce_shard_merge(stats, shards, m, n, lse, mws, sync=False)
        if st != lce.OK:
            raise lce.LceError(st, "lce_shard_merge")
        for q in range(shards):
            a, b = bounds[q], bounds[q + 1]
            st = lce.lce_shard_backward(H, W[a:b], y, m, lse, n, D, b - a, a, V, chunk,
                                        w.z_coef, 1.0, part, dW[a:b], 0, ws)
            if st != lce.OK:
                raise lce.LceError(st, "lce_shard_backward")
            if q == 0:
                dH.copy_(part)
            else:
                dH.add_(part)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    # the shard calls' target guards (their workspace) and the exchange's scalars
    st, _ = lce.lce_loss_fetch(ws)
    if st != lce.OK:
        raise lce.LceError(st, "lce_shard_forward / lce_shard_backward")
    st, out = lce.lce_loss_fetch(mws)
    if st != lce.OK:
        raise lce.LceError(st, "lce_shard_merge")
    return {"shards": shards, "bounds": bounds, "chunk_per_shard": chunk,
            "ms_per_step": round(ms, 4),
            "tokens_per_s": round(n / (ms / 1e3), 1), "loss": out.loss_mean}


def f16_measure(lce, torch, np, dev, w, steps: int):
    """The headline step with fp16 inputs (same shapes and draws, rounded to
    fp16; grad_out 65536 as an fp16 loss scale)."""
    import dataclasses
    from tests import synthetic as syn
    wf = dataclasses.replace(w, dtype="f16")
    log(f"bench: fp16 inputs for {w.name}: generating inputs")
    x = syn.ce_inputs(wf)
    n, D, V, chunk, z = w.n_tok, w.d_model, w.vocab, w.chunk, w.z_coef
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    m = torch.from_numpy(x.mask).to(dev) if x.mask is not None else None
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(V, D, dtype=torch.float32, device=dev)
    ws = torch.empty(lce.lce_workspace_bytes(n, D, V, chunk, H.dtype), dtype=torch.uint8,
                     device=dev)

    def step():
        st, _ = lce.lce_forward(H, W, y, m, n, D, V, chunk, z, lse, ws, sync=False)
        if st != lce.OK:
            raise lce.LceError(st, "lce_forward")
        st = lce.lce_backward(H, W, y, m, lse, n, D, V, chunk, z, 65536.0, dH, dW, 0, ws)
        if st != lce.OK:
            raise lce.LceError(st, "lce_backward")

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    st, out = lce.lce_loss_fetch(ws)
    flops = 8.0 * n * D * V
    return {"workload": w.name.replace("bf16", "f16"), "ms_per_step": round(ms, 4),
            "tokens_per_s": round(n / (ms / 1e3), 1),
            "tflops_8ndv": round(flops / (ms / 1e3) / 1e12, 2),
            "mfma_frac_8ndv": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "loss": out.loss_mean}


def step_runner(lce, w, H, W, y, m, lse, dH, dW, ws, grad_out=1.0):
    n, D = H.shape
    V = W.shape[0]

    def step(timer=None):
        st, _ = lce.lce_forward(H, W, y, m, n, D, V, w.chunk, w.z_coef, lse, ws, timer=timer,
                                sync=False)
        if st != lce.OK:
            raise lce.LceError(st, "lce_forward")
        st = lce.lce_backward(H, W, y, m, lse, n, D, V, w.chunk, w.z_coef, grad_out, dH, dW, 0,
                              ws, timer=timer)
        if st != lce.OK:
            raise lce.LceError(st, "lce_backward")
    return step


def per_step_ms(torch, step, steps: int):
    """Device time of each of `steps` steps (events between steps only)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def f64_sweep_measure(lce, torch, np, dev, steps: int):
    """The 2048 x 1024 x 151936 head in fp64 at chunk 128, 256 and 512 (step
    time, loss bit-identical across chunks) and chunk 1024, which the
    chunk*vocab budget refuses (587) before any work."""
    import dataclasses
    from tests import synthetic as syn
    w0 = syn.QWEN_F64
    log(f"bench: fp64 chunk sweep {w0.name}: generating inputs")
    x = syn.ce_inputs(w0)
    n, D, V = w0.n_tok, w0.d_model, w0.vocab
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    lse = torch.empty(n, dtype=torch.float64, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(V, D, dtype=torch.float64, device=dev)
    flops = 8.0 * n * D * V
    res = {"workload": w0.name, "peak_tflops": PEAK_F64_TFLOPS, "chunks": {}}
    losses = []
    for chunk in (128, 256, 512, 1024):
        nb = lce.lce_workspace_bytes(n, D, V, chunk, torch.float64)
        if nb < 0:
            st, _ = lce.lce_forward(H, W, y, None, n, D, V, chunk, 0.0, lse,
                                    torch.empty(1024, dtype=torch.uint8, device=dev))
            res["chunks"][str(chunk)] = {"status": int(-nb), "forward_status": int(st)}
            continue
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        step = step_runner(lce, dataclasses.replace(w0, chunk=chunk), H, W, y, None, lse, dH, dW,
                           ws)
        step()
        torch.cuda.synchronize()
        t = per_step_ms(torch, step, steps)
        st, out = lce.lce_loss_fetch(ws)
        losses.append(out.loss_mean)
        med = float(np.median(t))
        res["chunks"][str(chunk)] = {
            "status": int(st), "ms_median": round(med, 3), "ms_min": round(float(np.min(t)), 3),
            "tflops_8ndv": round(flops / (med / 1e3) / 1e12, 2),
            "frac_8ndv": round(flops / (med / 1e3) / 1e12 / PEAK_F64_TFLOPS, 4),
            "loss": out.loss_mean, "workspace_bytes": nb}
        del ws
    res["loss_bit_identical_across_chunks"] = len(set(losses)) == 1
    del H, W, dW, dH
    torch.cuda.empty_cache()
    return res


def large_head_measure(lce, torch, np, dev, steps: int):
    """The 8192 x 4096 x 128256 bf16 head (Zipf targets, chunk 512, z
    1e-4): the same step as the headline, per-step device time."""
    from tests import synthetic as syn
    w = syn.LARGE_BF16
    log(f"bench: {w.name}: generating inputs")
    x = syn.ce_inputs(w)
    n, D, V = w.n_tok, w.d_model, w.vocab
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(V, D, dtype=torch.float32, device=dev)
    ws = torch.empty(lce.lce_workspace_bytes(n, D, V, w.chunk, H.dtype), dtype=torch.uint8,
                     device=dev)
    step = step_runner(lce, w, H, W, y, None, lse, dH, dW, ws)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t = per_step_ms(torch, step, steps)
    st, out = lce.lce_loss_fetch(ws)
    med = float(np.median(t))
    flops = 8.0 * n * D * V
    res = {"workload": w.name, "status": int(st), "ms_median": round(med, 3),
           "ms_min": round(float(np.min(t)), 3), "tokens_per_s": round(n / (med / 1e3), 1),
           "tflops_8ndv": round(flops / (med / 1e3) / 1e12, 2),
           "mfma_frac_8ndv": round(flops / (med / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "mfma_frac_6ndv": round(0.75 * flops / (med / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "loss": out.loss_mean}
    del H, W, dW, dH, ws
    torch.cuda.empty_cache()
    return res


def single_call_measure(lce, torch, np, dev, steps: int):
    """lce_forward_backward (the whole batch in one chunk) against
    lce_forward + lce_backward (8nDV) on the same bf16 inputs with the
    151936-row vocabulary, z 1e-4, 5% masked.  Where the call's cost model
    keeps the logits it does 6nDV; elsewhere it runs the two-call algorithm
    (keeps_logits 0)."""
    from tests import synthetic as syn
    out = []
    for n, D in ((256, 1024), (512, 1024), (512, 4096)):
        V, chunk, z = 151936, n, 1e-4
        log(f"bench: single call {n} x {D} x {V}: generating inputs")
        x = syn.ce_inputs(syn.QWEN_BF16, n_tok=n, d_model=D, vocab=V, seed=7)
        H, W = x.hidden.to(dev), x.weight.to(dev)
        y = torch.from_numpy(x.targets).to(dev)
        m = torch.from_numpy(syn.exact_mask(np.random.default_rng(7), n, 0.05)).to(dev)
        lse = torch.empty(n, dtype=torch.float32, device=dev)
        dH = torch.empty_like(H)
        dW = torch.empty(V, D, dtype=torch.float32, device=dev)
        ws1 = torch.empty(lce.lce_forward_backward_workspace_bytes(n, D, V, chunk, H.dtype),
                          dtype=torch.uint8, device=dev)
        ws2 = torch.empty(lce.lce_workspace_bytes(n, D, V, chunk, H.dtype), dtype=torch.uint8,
                          device=dev)

        def single():
            st, _ = lce.lce_forward_backward(H, W, y, m, n, D, V, chunk, z, 1.0, lse, dH, dW, 0,
                                             ws1, sync=False)
            if st != lce.OK:
                raise lce.LceError(st, "lce_forward_backward")

        def two():
            st, _ = lce.lce_forward(H, W, y, m, n, D, V, chunk, z, lse, ws2, sync=False)
            if st != lce.OK:
                raise lce.LceError(st, "lce_forward")
            st = lce.lce_backward(H, W, y, m, lse, n, D, V, chunk, z, 1.0, dH, dW, 0, ws2)
            if st != lce.OK:
                raise lce.LceError(st, "lce_backward")

        # Both variants warm up together (the clock settles under the load),
        # then run in alternating blocks; each block's wall time over its
        # steps, median over the blocks, so that neither variant is the one
        # timed on a cold clock.
        fs = {"single": single, "two_calls": two}
        for _ in range(max(3, steps // 2)):
            single()
            two()
        torch.cuda.synchronize()
        blocks = {k: [] for k in fs}
        for _ in range(5):
            for name, f in fs.items():
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(steps):
                    f()
                torch.cuda.synchronize()
                blocks[name].append((time.perf_counter() - t0) / steps * 1e3)
        ms = {k: float(np.median(v)) for k, v in blocks.items()}
        f2 = 2.0 * n * D * V
        out.append({"n_tok": n, "d_model": D, "vocab": V, "chunk": chunk,
                    "keeps_logits": lce.lce_forward_backward_keeps_logits(n, D, V, chunk,
                                                                          H.dtype),
                    "single_ms": round(ms["single"], 4), "two_calls_ms": round(ms["two_calls"], 4),
                    "speedup": round(ms["two_calls"] / ms["single"], 4),
                    "single_tflops_6ndv": round(3 * f2 / (ms["single"] / 1e3) / 1e12, 2),
                    "two_calls_tflops_8ndv": round(4 * f2 / (ms["two_calls"] / 1e3) / 1e12, 2),
                    "workspace_bytes": int(ws1.numel())})
        del H, W, dW, ws1, ws2
        torch.cuda.empty_cache()
    return out


def cpu_model_name() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" if absent)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Samples the GPU's current graphics clock (MHz) and socket power (W)
    through amdsmi from a background thread while the caller keeps the GPU
    busy; best effort (no samples when amdsmi cannot be initialised)."""

    def __init__(self, period_s: float = 0.005):
        import threading
        self.period = period_s
        self.clk, self.power = [], []
        self._stop = threading.Event()
        self._thread = None
        self.error = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:          # noqa: BLE001 - optional telemetry
            self._smi = None
            self.error = f"{type(e).__name__}: {e}"

    def _run(self):
        smi = self._smi
        while not self._stop.is_set():
            try:
                c = smi.amdsmi_get_clock_info(self._h, smi.AmdSmiClkType.GFX)
                self.clk.append(float(c.get("clk", c.get("cur_clk", 0))))
            except Exception as e:      # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            try:
                p = smi.amdsmi_get_power_info(self._h)
                v = p.get("current_socket_power", p.get("average_socket_power"))
                if isinstance(v, (int, float)):
                    self.power.append(float(v))
            except Exception:           # noqa: BLE001
                pass
            time.sleep(self.period)

    def __enter__(self):
        import threading
        if self._smi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:           # noqa: BLE001
                pass

    def summary(self) -> dict:
        import numpy as np
        out = {"samples": len(self.clk)}
        if self.clk:
            # the telemetry lags the load: keep the second half of the samples
            c = np.array(self.clk[len(self.clk) // 2:])
            out.update({"gfx_mhz_median": float(np.median(c)), "gfx_mhz_min": float(np.min(c)),
                        "gfx_mhz_max": float(np.max(c))})
        if self.power:
            pw = np.array(self.power[len(self.power) // 2:])
            out["socket_power_w_median"] = float(np.median(pw))
        if self.error:
            out["error"] = self.error
        return out


def mfma_ceiling_measure(torch, np, dev, fwd_tflops=None):
    """A practical ceiling for bf16 matrix work on this part: torch.matmul
    (hipBLASLt) on random bf16 8192 x 8192 x 8192 operands, timed with events
    over a loop of about two seconds, with the graphics clock and socket power
    sampled meanwhile; the same on constant operands (less switching activity
    per MFMA) for contrast.  The nominal peak assumes 2400 MHz."""
    N = 8192
    out = {"shape": [N, N, N], "dtype": "bf16", "library": "torch.matmul (hipBLASLt)",
           "nominal_peak_tflops": PEAK_BF16_TFLOPS}
    for kind in ("random", "constant"):
        if kind == "random":
            a = torch.randn(N, N, device=dev, dtype=torch.bfloat16)
            b = torch.randn(N, N, device=dev, dtype=torch.bfloat16)
        else:
            a = torch.full((N, N), 0.5, device=dev, dtype=torch.bfloat16)
            b = torch.full((N, N), 0.25, device=dev, dtype=torch.bfloat16)
        c = torch.empty(N, N, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        iters = 40
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # about 1.5 s of back-to-back products; the telemetry lags, so the
        # sampler's summary keeps the later samples, and the time is that of
        # the last round
        with ClockSampler() as cs:
            t_end = time.perf_counter() + 1.5
            while time.perf_counter() < t_end:
                e0.record()
                for _ in range(iters):
                    torch.matmul(a, b, out=c)
                e1.record()
                torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        tf = 2.0 * N ** 3 / (ms / 1e3) / 1e12
        rec = {"ms": round(ms, 4), "tflops": round(tf, 1),
               "frac_of_nominal": round(tf / PEAK_BF16_TFLOPS, 4), "clock": cs.summary()}
        mhz = rec["clock"].get("gfx_mhz_median")
        if mhz:
            rec["peak_at_measured_clock_tflops"] = round(PEAK_BF16_TFLOPS * mhz / 2400.0, 1)
        out[kind] = rec
        del a, b, c
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, x, tokens: int):
    """The oracle, as it stands, on the first `tokens` tokens of the workload:
    forward (all tokens of the prefix) + backward (d_hidden of the prefix and
    every d_weight row)."""
    import numpy as np
    import oracle

    H = x.hidden[:tokens].to(dtype=__import__("torch").float64).numpy()
    W = x.weight64()
    y = x.targets[:tokens]
    m = x.mask[:tokens] if x.mask is not None else None
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    r = oracle.fused_forward(H, W, y, mask=m, chunk=w.chunk, z_coef=w.z_coef, nthreads=threads)
    oracle.backward(H, W, y, r["lse"], mask=m, z_coef=w.z_coef, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model_name(),
            "sample": f"first {tokens} tokens of the {w.n_tok}-token batch, full vocab "
                      f"{w.vocab} and d_model {w.d_model}: fp64 forward + backward "
                      f"(d_hidden of the sample, all d_weight rows), {dt:.2f} s",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen_bf16",
                    choices=["qwen_bf16", "large_bf16", "qwen_f64"])
    ap.add_argument("--cpu-tokens", type=int, default=768)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device twice and exit (the known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--single-call-only", action="store_true",
                    help="only time lce_forward_backward against the two calls (512 tokens, "
                         "d_model 1024 and 4096) and print that record")
    ap.add_argument("--logits-in-only", action="store_true",
                    help="only time the logits-in kernels (distillation and label CE at "
                         "4096 x 151936 bf16) and print that record")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true")
    ap.add_argument("--no-shards", action="store_true",
                    help="skip the vocabulary-shard measurement")
    ap.add_argument("--no-distill", action="store_true",
                    help="skip the side measurements (vocabulary shards, distillation and label CE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.single_call_only:
        from lm_head_linear_amd import lce
        lce.lib()
        res = single_call_measure(lce, torch, np, torch.device("cuda:0"), args.steps)
        print(json.dumps({"single_call": res}), flush=True)
        return

    if args.logits_in_only:
        from lm_head_linear_amd import lce
        lce.lib()
        dev = torch.device("cuda:0")
        res = {"distill": distill_measure(lce, torch, np, dev, args.steps),
               "label_ce": label_measure(lce, torch, np, dev, args.steps)}
        print(json.dumps(res), flush=True)
        return

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        # the same copy timed: read + write bytes over time, a practical HBM ceiling
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        gbs = 2 * nbytes * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
        print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 2,
                          "copy_read_write_GBs": round(gbs, 1)}), flush=True)
        return

    from lm_head_linear_amd import lce
    from tests import synthetic as syn

    w = {"qwen_bf16": syn.QWEN_BF16, "large_bf16": syn.LARGE_BF16,
         "qwen_f64": syn.QWEN_F64}[args.workload]
    dev = torch.device("cuda:0")
    log(f"bench: workload {w.name}: generating inputs")
    x = syn.ce_inputs(w)
    n, D, V, chunk, z = w.n_tok, w.d_model, w.vocab, w.chunk, w.z_coef
    H, W = x.hidden.to(dev), x.weight.to(dev)
    y = torch.from_numpy(x.targets).to(dev)
    m = torch.from_numpy(x.mask).to(dev) if x.mask is not None else None
    acc_dt = torch.float64 if H.dtype == torch.float64 else torch.float32
    lse = torch.empty(n, dtype=acc_dt, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(V, D, dtype=acc_dt, device=dev)
    ws_bytes = lce.lce_workspace_bytes(n, D, V, chunk, H.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    # forward and backward without a host round trip (neither call waits for
    # the device); the loss scalars and the target guard's verdict stay in the
    # workspace until lce_loss_fetch
    step = step_runner(lce, w, H, W, y, m, lse, dH, dW, ws)

    def fetch():
        st, out = lce.lce_loss_fetch(ws)
        if st != lce.OK:
            raise lce.LceError(st, "lce_loss_fetch")
        return out

    log(f"bench: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    fetch()
    torch.cuda.synchronize()

    # Timed pass: K steps, nothing recorded between the kernels.
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    out = fetch()
    ms_per_step = 1e3 * wall / args.steps
    peak_extra = torch.cuda.max_memory_allocated() - mem0
    log(f"bench: {ms_per_step:.3f} ms/step wall, {gpu_ms / args.steps:.3f} ms/step events, "
        f"loss {out.loss_mean:.6f}")

    # Per-step pass: the same K steps with an event between consecutive steps
    # (median and min of the per-step device times).
    steps_ms = per_step_ms(torch, step, args.steps)
    fetch()
    log(f"bench: per-step median {np.median(steps_ms):.4f} ms, min {np.min(steps_ms):.4f} ms")

    # Kernel pass: the same K steps again with HIP events around every kernel
    # launch (on the launch stream); the events add idle time between kernels,
    # so this pass gives kernel durations only, never the step time.
    timer = None
    if not args.no_kernel_events:
        timer = lce.KernelTimer(ALL_KINDS, capacity=args.steps * 32)
        log(f"bench: kernel pass, {args.steps} steps with per-kernel events")
        for _ in range(args.steps):
            step(timer)
        torch.cuda.synchronize()

    # Split pass: forward and backward device time per step (events between
    # the calls only); then the same with L2 and the Infinity Cache flushed by
    # a 512 MB scratch write before every step ("cold").
    split = {"fwd_ms": [], "bwd_ms": [], "cold_fwd_ms": [], "cold_bwd_ms": []}
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for i in range(2 * args.steps):
        cold = i >= args.steps
        if cold:
            scratch.fill_(i & 0xff)
        ea, eb, ec = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        ea.record()
        st, _ = lce.lce_forward(H, W, y, m, n, D, V, chunk, z, lse, ws, sync=False)
        eb.record()
        st2 = lce.lce_backward(H, W, y, m, lse, n, D, V, chunk, z, 1.0, dH, dW, 0, ws)
        ec.record()
        torch.cuda.synchronize()
        if st != lce.OK or st2 != lce.OK:
            raise lce.LceError(st if st != lce.OK else st2, "split pass")
        split["cold_fwd_ms" if cold else "fwd_ms"].append(ea.elapsed_time(eb))
        split["cold_bwd_ms" if cold else "bwd_ms"].append(eb.elapsed_time(ec))
    del scratch
    split = {k: {"median": round(float(np.median(v)), 4), "min": round(float(np.min(v)), 4)}
             for k, v in split.items()}

    flop_gemm = 2.0 * n * D * V                  # one GEMM pass over every (token, vocab) pair
    f8 = 4 * flop_gemm                            # forward + recompute + dH + dW
    f6 = 3 * flop_gemm
    tokens_per_s = n / (ms_per_step / 1e3)
    peak = PEAK_F64_TFLOPS if w.dtype == "f64" else PEAK_BF16_TFLOPS

    kernels = {}
    roof = None
    if timer is not None:
        for k in ALL_KINDS:
            d = timer.durations_ms(k)
            if d:
                kernels[k] = {"launches_per_step": len(d) / args.steps,
                              "avg_ms": float(np.mean(d)), "ms_per_step": float(np.sum(d)) / args.steps}
        dom = max((k for k in GEMM_KINDS if k in kernels), key=lambda k: kernels[k]["ms_per_step"])
        kd = kernels[dom]
        per_launch_flops = GEMM_PASSES[dom] * flop_gemm / kd["launches_per_step"]
        achieved = per_launch_flops / (kd["avg_ms"] / 1e3) / 1e12
        for k in GEMM_KINDS:
            if k in kernels:
                kernels[k]["tflops"] = (GEMM_PASSES[k] * flop_gemm /
                                        (kernels[k]["ms_per_step"] / 1e3) / 1e12)
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_from_profiles(w.name, dom),
                "kernel": dom, "flops_per_launch": per_launch_flops, "avg_launch_ms": kd["avg_ms"]}

    f16 = None
    if w.dtype == "bf16" and not (args.no_distill or args.no_shards):
        f16 = f16_measure(lce, torch, np, dev, w, args.steps)

    single = None
    if w.dtype == "bf16" and not (args.no_distill or args.no_shards):
        single = single_call_measure(lce, torch, np, dev, args.steps)

    shard = None
    if w.dtype == "bf16" and not (args.no_distill or args.no_shards):
        log("bench: the same step in 4 vocabulary shards")
        shard = shard_measure(lce, torch, np, dev, w, H, W, y, m, args.steps, 4)
        shard["vs_unsharded"] = round(ms_per_step / shard["ms_per_step"], 4)

    distill = label = None
    if not args.no_distill and w.dtype == "bf16":
        distill = distill_measure(lce, torch, np, dev, args.steps)
        label = label_measure(lce, torch, np, dev, args.steps)

    f64_sweep = large = ceiling = None
    if w.dtype == "bf16" and not args.no_distill:
        f64_sweep = f64_sweep_measure(lce, torch, np, dev, max(3, args.steps // 5))
        large = large_head_measure(lce, torch, np, dev, max(5, args.steps // 4))
        log("bench: practical bf16 MFMA ceiling (torch.matmul 8192^3) with clock sampling")
        ceiling = mfma_ceiling_measure(torch, np, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle baseline on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(w, x, args.cpu_tokens)
        cpu.pop("seconds", None)

    res = {
        "metric": "fused linear-CE fwd+bwd tokens/s and % MFMA peak at 2048x1024x151936 bf16",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_median": round(float(np.median(steps_ms)), 4),
        "step_ms_min": round(float(np.min(steps_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f64",
        "data": "synthetic",
        "config": {"workload": w.name, "n_tok": n, "d_model": D, "vocab": V, "chunk": chunk,
                   "z_coef": z, "mask_frac": w.mask_frac, "targets": w.targets},
        "tflops_8ndv": round(f8 / (ms_per_step / 1e3) / 1e12, 2),
        "mfma_frac_8ndv": round(f8 / (ms_per_step / 1e3) / 1e12 / peak, 4),
        "tflops_6ndv": round(f6 / (ms_per_step / 1e3) / 1e12, 2),
        "mfma_frac_6ndv": round(f6 / (ms_per_step / 1e3) / 1e12 / peak, 4),
        "gpu_ms_per_step_events": round(gpu_ms / args.steps, 4),
        "workspace_bytes": ws_bytes,
        "peak_extra_bytes": int(peak_extra),
        "fwd_bwd_split": split,
        "kernels": kernels,
        "roofline": roof,
        "distill": distill,
        "label_ce": label,
        "vocab_shards": shard,
        "f16_inputs": f16,
        "single_call": single,
        "f64_chunk_sweep": f64_sweep,
        "large_head": large,
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
