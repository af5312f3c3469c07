"""Write the oracle's per-token forward statistics for the large workloads.

Calls only the CPU oracle (and the seeded generators): for each named workload it
stores fp32 log-prob, log-sum-exp and entropy of every token, which the GPU
tests use to form old/ref log-probs (fp32(current) + noise, the generators'
recipe) and as expected values. Usage:

    python tests/golden/make_golden.py gmpo_kl_bf16_b8_t2048 gspo_token_entropy_bf16_b2_t32768

Output: tests/golden/fwd_<workload>.npz (arrays logp, lse, entropy; fp32).
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def main(names):
    for c in names:
        spec = synth.WORKLOADS[c]
        t0 = time.time()
        h, _ = synth.hidden(spec)
        W, _ = synth.weight(spec)
        b, _ = synth.bias(spec)
        y = synth.targets(spec)
        W64 = W.astype(np.float64)
        b64 = None if b is None else b.astype(np.float64)
        N = spec.N
        lp = np.empty(N, np.float32)
        lse = np.empty(N, np.float32)
        ent = np.empty(N, np.float32)
        step = 2048
        for r0 in range(0, N, step):
            r1 = min(N, r0 + step)
            f = oracle.forward_rows(h[r0:r1], W64, b64, spec.temperature, y[r0:r1])
            lp[r0:r1], lse[r0:r1], ent[r0:r1] = f["logp"], f["lse"], f["entropy"]
            print(f"{c}: {r1}/{N} rows, {time.time() - t0:.0f} s", flush=True)
        out = os.path.join(HERE, f"fwd_{c}.npz")
        np.savez_compressed(out, logp=lp, lse=lse, entropy=ent)
        print(f"wrote {out} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["gmpo_kl_bf16_b8_t2048", "gspo_token_entropy_bf16_b2_t32768"])
