"""fp64 CPU oracle for the TurboQuant key path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What it computes follows the pages, in their order and notation:

* the randomized Hadamard rotation R = H_d D / sqrt(d), with H_d built by the
  Sylvester recursion and D a Rademacher diagonal
  [ICLR 2026 paper digest (0h-n0), "Step 1: PolarQuant", eq. for R];
* unit normalisation with the norm kept on the side and the zero-vector rule
  [same page, "実装の擬似コード" (turboquant_encode) and "実装のポイント",
  norm storage];
* a (b-1)-bit Lloyd-Max scalar quantizer for the N(0, 1/d) law of each
  rotated coordinate [same page, Step 1 / Theorem 1; Qiita explainer,
  "Stage 1" step 3];
* a 1-bit QJL sketch sign(S r) of the residual r = k - k_mse
  [Qiita explainer, "Stage 2: QJL", estimator equation; ai.spot.hk article,
  "無偏內積估計" (TURBOQUANT_prod = (b-1)-bit MSE stage + 1-bit QJL)];
* the asymmetric estimator
  <q,k> ~ <q,k_mse> + ||r|| sqrt(pi/2)/m <S q, sign(S r)>
  [Qiita explainer, "Stage 2: QJL", estimator equation].

Everything is float64 numpy, with a dense explicit rotation matrix (never a
butterfly), residuals formed in the original domain, and its own
implementation of the seed -> (delta, S) generator and of the packed layout.

Parity pins (tests/test_oracle_pins.py) tie every function to something
other than itself: closed forms, textbook Lloyd-Max tables, brute force on
tiny inputs, Monte-Carlo unbiasedness, the Shannon-bound ratio, and the byte
table printed on the Qiita explainer.  Functions with no independent pin
say "parity unpinned" in their docstring.
"""

from .turboquant import *  # noqa: F401,F403
