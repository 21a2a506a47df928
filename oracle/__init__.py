"""CPU oracle for the split-invariant logprob forward -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP kernels are checked
against. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or run it; the product path
(``split_invariant_deterministic_amd``) never does, and this package imports
nothing from it. The two share no kernels, headers, helpers, tables or
constant generators; only seeded input generators (which hold none of the
method's arithmetic) feed both sides, and they are never imported here.

What the oracle computes, per step:

* the plain mathematical definition of each step in float64 from the same
  bf16 inputs (GEMM sums, RMSNorm, log-softmax, attention, MoE FFN), and
* a step-by-step replay of the parts of the rounding schedule that a CPU can
  reproduce bit for bit: fp32 leaf-tree additions (IEEE round-to-nearest-even
  float32 adds in numpy, no contraction), the bf16 boundary cast, and the
  chunk / split boundaries.

Sources, cited by page title and section:

* [IsoExec] vllm.ai blog "IsoExec: Unified Execution to Eliminate
  Trainer-Inference Mismatch in SkyRL"
* [NovaSky] alphasignal.ai "NovaSky's IsoExec Fixes the Hidden Math Bug
  Corrupting AI Training Runs"
* [RLK] "Reinforcement Learning Post-Training for Large Models: How RL-Kernel
  Completely Eliminates Train-Inference LogP Discrepancy"
* [VeXact] arXiv 2605.14220 "Diagnosing Training Inference Mismatch in LLM
  Reinforcement Learning"

Parity status of each function is stated in its module docstring. The bits
of a single MFMA leaf chain and of the GPU's exp2/sum order are
hardware-defined and therefore "parity unpinned" bitwise; they are pinned by
error bounds here and by GPU-vs-GPU invariance in the tests.
"""

from . import numerics, tree, gemm, rmsnorm, logprob, attention, moe  # noqa: F401
