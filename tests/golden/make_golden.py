"""Writes the stored expected values under tests/golden/ from the CPU oracle.

Run from the repository root:  python tests/golden/make_golden.py
Inputs come from the seeded generators; every expected value comes from
``oracle/`` only (never from the HIP path).
"""
import hashlib
import json
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import gemm as ogemm, logprob as olp, rmsnorm as orms  # noqa: E402
from split_invariant_deterministic_amd import synth  # noqa: E402


def main():
    t = synth.tiny(0)
    hashes = {k: hashlib.sha256(t[k].contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
              for k in ("x", "W", "targets")}
    json.dump(hashes, open(os.path.join(HERE, "synth_hashes.json"), "w"), indent=1)

    x = t["x"].float().numpy()
    W = t["W"].float().numpy()
    y = orms.rmsnorm(x, t["gamma"].float().numpy(), 1e-6)          # bf16 values
    logits_tree = ogemm.gemm_tree(y, W, 4, "fp32")                   # leaf/tree schedule
    logits_plain = ogemm.gemm(y, W, "fp64")
    lp = olp.logprob(logits_tree, t["targets"].numpy())
    np.savez(os.path.join(HERE, "tiny_expected.npz"), rms_y=y.astype(np.float32),
             logits_tree=logits_tree, logits_plain=logits_plain, logprob=lp)
    print("wrote synth_hashes.json and tiny_expected.npz")


if __name__ == "__main__":
    main()
