"""Write the router bias of the skewed workloads (tests/golden/zipf_bias_*.txt).

The skewed workloads ask for router logits with a per-expert bias chosen so
that expert popularity follows Zipf(s): the probability that a token picks
expert e is proportional to (e+1)^-s, capped at 1 and summing to k.  The
bias is an INPUT of both the HIP path and the oracle.  It is calibrated here
on a separate seeded batch of calibration tokens with the oracle's own logits
and top-k (this script calls nothing but oracle/ and the input generator):
  b <- 0;  repeat 100 times:  f_e = fraction of calibration tokens choosing e
  under logits z + b;  b_e += 0.5 sigma_z (ln p_e - ln max(f_e, 0.5/n)).
Run:  python tests/golden/make_zipf_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from combine_router_top_expert_amd import synth  # noqa: E402


def calibrate(w, n_cal=8192, iters=100):
    _, xv = synth.gen_calibration_tokens(w, n_cal)
    _, wrv = synth.gen_router(w)
    z0 = oracle.logits(xv, wrv, None, w.prec).astype(np.float32)  # fp32 chain, no bias
    target = synth.zipf_popularity(w.E, w.k, w.zipf_s)
    sigma = float(z0.std())
    b = np.zeros(w.E, np.float32)
    f = None
    for _ in range(iters):
        z = (z0 + b[None, :]).astype(np.float64)  # one fp32 add of the bias, as the layer does
        idx = oracle.topk(z, w.k)
        f = np.bincount(idx.ravel(), minlength=w.E) / n_cal
        step = 0.5 * sigma * (np.log(target) - np.log(np.maximum(f, 0.5 / n_cal)))
        b = (b + step).astype(np.float32)
    return b, f, target


def main():
    for name in ("C3", "C5"):
        w = synth.WORKLOADS[name]
        b, f, target = calibrate(w)
        path = synth.bias_file(w)
        with open(path, "w") as fh:
            fh.write(f"# router bias for Zipf({w.zipf_s}) popularity, E={w.E} k={w.k} d={w.d} "
                     f"router std {w.router_std:.6g}\n")
            fh.write("# written by tests/golden/make_zipf_bias.py (oracle logits + top-k on "
                     "8192 calibration tokens)\n")
            fh.write("# realised pick fraction per expert (first 8): "
                     + " ".join(f"{v:.4f}" for v in f[:8]) + "\n")
            fh.write("# target pick fraction per expert  (first 8): "
                     + " ".join(f"{v:.4f}" for v in target[:8]) + "\n")
            for v in b:
                fh.write(float(v).hex() + "\n")
        print(name, path, "max |f - target| =", float(np.abs(f - target).max()))


if __name__ == "__main__":
    main()
