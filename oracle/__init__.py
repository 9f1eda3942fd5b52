"""CPU oracle for the outlier-aware quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``outlier_aware_bit_amd``) and never imports it.

Plain, slow, obviously-correct NumPy.  Each function cites the passage of the
pages it follows (page title + section).  Conventions:

* Integer GEMMs run as float64 matrix products of integer-valued arrays; every
  partial sum stays far below 2**53, so the result is the exact integer
  (asserted in ``gemm.exact_int_matmul``).
* Wherever a float decides an integer code (a quantizer), the decision is
  taken in IEEE float32 with one rounding per operation, exactly as the
  kernels do; ``np.rint`` rounds half to even.
* Float outputs (dequantized Y) are computed in float64.

Modules:
  hadamard  -- Sylvester / partially random Hadamard matrices, block transform
  quant     -- activation and weight quantizers (symmetric int8/int4, per-group,
               asymmetric int4 with zero point, the fused dequant-quant)
  gemm      -- integer accumulators and dequantized outputs of W8A8, W4A8, W4A4
  quaff     -- sparse outlier compensation and the momentum scale update
  layer     -- whole-layer forward passes composed from the above
  pca       -- OffQ's Top-1 PCA concentration (extreme tokens, covariance,
               leading eigenvector, Householder rotation of acts and weights)

Parity pins: every public function is pinned in ``tests/test_oracle_*.py``
against closed forms, brute force in exact Python integers / fractions,
library routines, or hand-worked examples in ``tests/golden/``.
"""
from . import hadamard, quant, gemm, quaff, layer, pca  # noqa: F401
