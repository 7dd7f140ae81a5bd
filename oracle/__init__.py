"""fp64 CPU oracle for the GPTQ layer-quantization path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The product (the HIP library and its Python binding) never imports this
package and shares no code, header, table or helper with it; both sides only
share the seeded input generators in ``synth``.

What it computes, and where each step is defined (pages cited by title and
section; "the pages" are the five web pages on GPTQ this path is built from):

* ``quantizer`` -- the uniform affine / symmetric quantizers, per-group
  parameters, round-to-nearest (RTN) baseline and the packed 4-bit storage
  format ("INT4 and GPTQ Quantization": Uniform INT4 Quantization, Group
  Quantization; "Quantization (INT8, INT4, GPTQ)": Deriving the scale and
  zero-point; "GPTQ: Mathematical Foundations ...": Quantization Formats and
  Group Size, Inference Execution).
* ``hessian`` -- H = 2 X Xᵀ ("GPTQ: Mathematical Foundations ...": Second-Order
  Taylor Expansion and the Hessian).
* ``prepare`` -- dead-channel fix, relative diagonal damping, act-order
  permutation, inverse Hessian and its upper Cholesky factor
  ("GPTQ: Mathematical Foundations ...": Hessian Damping and Numerical
  Regularization, Activation Ordering, Cholesky Decomposition and
  Pre-computation, GPTQ Algorithm Execution Walkthrough).
* ``gptq`` -- the fixed-order blocked column sweep with OBS compensation and
  lazy block updates ("GPTQ: Mathematical Foundations ...": The GPTQ
  Algorithmic Innovations 1-3), including a follow mode that checks another
  implementation's near-tie rounding decisions.
* ``obs`` -- the same greedy-in-fixed-order OBS process written with the
  explicit inverse-Hessian downdate ("GPTQ: Mathematical Foundations ...":
  Lagrangian Derivation, Recursive Inverse Hessian Updating), used to pin the
  Cholesky form.
* ``obq`` -- Optimal Brain Quantization: the same OBS step with the greedy
  order (smallest saliency first, every row its own order), the comparator
  for GPTQ's fixed order ("GPTQ: Mathematical Foundations ...": OBS and OBQ,
  The Computational Bottleneck of OBQ, The GPTQ Algorithmic Innovations 1).
* ``w4a16`` -- inference with the exported weights: dequantize to the
  activations' 16-bit format and multiply ("GPTQ: Mathematical Foundations
  ...", Inference Execution and Modern Kernel Architectures).
* ``metrics`` -- layer output error, brute-force optimum on tiny layers, and
  the loss identity that follows from the OBS error penalty.

Every floating-point step is fp64.  Inputs arrive as stored bits (fp32 or
bf16) and are widened exactly.
"""
from .quantizer import (  # noqa: F401
    asym_params, asym_quantize, sym_params, sym_quantize, rtn_grouped,
    pack_codes, unpack_codes, bits_per_weight, Params,
    pack_dense, unpack_dense, fp16_bits, stored_bits_per_weight,
)
from .hessian import hessian  # noqa: F401
from .prepare import prepare, dead_fix, act_order_perm, inverse_cholesky_upper  # noqa: F401
from .gptq import gptq_sweep, gptq_layer, FollowReport  # noqa: F401
from .obs import obs_sequential  # noqa: F401
from .obq import obq_row, obq_layer  # noqa: F401
from . import w4a16  # noqa: F401
from .metrics import layer_error, layer_error_rows, brute_force_row, loss_identity_rhs  # noqa: F401
