"""CPU oracle for the MXFP4 + SiTU routed-MoE expert layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy restatement of what the layer computes.  It exists to check the HIP path
and to serve as the timed CPU baseline.  Only the test suite, the smoke entry
point and the benchmark's ``cpu_baseline`` leg may import it; the product path
(``block_scaled_mxfp4_amd``) never does, and this package imports nothing from
the product path.

Sources (cited by page title and section throughout):

* "TokenSpeed SiTU" (PyPI page of tokenspeed-situ), sections "Activation
  precision (w4a16 vs w4a8)", "Supported contract" and "Runtime API": the
  shard contract, the two activation modes and the partial output.
* "bring up Kimi K3 NVFP4 with CUTLASS and cuteDSL MegaMoE SiTU"
  (TensorRT-LLM pull request 17865): the review of
  ``test_kimi_k3_situ_moe.py`` that shows the golden routed-MoE skeleton and
  the SiTU formula, and the MegaMoE commit message ("SiTU in the kernel") that
  gives the tanh/sigmoid identity and K3's constants beta=4, linear beta=25.
* "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT -- Kimi-K3 SiTU" (xorl-wheels
  release notes), section "Changes since 875b7d7": per-expert beta and linear
  beta, and the rescale of the up half by its alpha before the tanh.
* OCP Microscaling Formats (MX) Specification v1.0 (external; the pages name
  the formats but never print them): E2M1, E4M3, E8M0 and the block-scale rule.

Parity status of each function is stated in its module's header.
"""

from . import formats, moe  # noqa: F401
