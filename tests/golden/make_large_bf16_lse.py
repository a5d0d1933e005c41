"""Writes large_head_bf16_8192x4096x128256_lse.txt: the oracle's per-token
log-sum-exp and loss scalars for the 8192 x 4096 x 128256 bf16 workload
(Zipf 1.1 targets, chunk 512, z 1e-4; the generator in tests/synthetic.py).

Only oracle/ computes here (fp64 C, all host cores); the full forward takes
minutes on a CPU, which is why its result is stored.  Run from the repository
root:  python3 tests/golden/make_large_bf16_lse.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tests import synthetic as syn  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                   "large_head_bf16_8192x4096x128256_lse.txt")


def main():
    w = syn.LARGE_BF16
    x = syn.ce_inputs(w)
    H, W = x.hidden64(), x.weight64()
    r = oracle.fused_forward(H, W, x.targets, mask=x.mask, chunk=w.chunk, z_coef=w.z_coef,
                             nthreads=oracle.default_threads())
    assert r["status"] == 580, r["status"]
    with open(OUT, "w") as f:
        f.write(f"# oracle.fused_forward on {w.name}: seed {w.seed}, chunk {w.chunk}, "
                f"z_coef {w.z_coef}, targets {w.targets}\n")
        f.write("# written by tests/golden/make_large_bf16_lse.py (oracle only)\n")
        f.write(f"loss_sum {r['loss_sum']!r}\nz_sum {r['z_sum']!r}\nn_counted {r['n_counted']}\n")
        f.write("lse\n")
        for v in r["lse"]:
            f.write(f"{float(v)!r}\n")


if __name__ == "__main__":
    main()
