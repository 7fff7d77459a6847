"""CPU oracle for batched draft-token verification and the online acceptance
estimator.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and the
two share no code: no kernels, headers, helpers, tables or pre/post-processing.
Only the seeded input generators in ``synth`` feed both.

Everything here is plain float64 numpy, written step by step in the order the
pages give the method, with no blocking or fusion.  Pages cited:

[CS]  "Speculative Decoding: Draft, EAGLE, MTP" - cheat sheet (nextadmin.net,
      Persian), sections "One speculative step", "Algorithm loop in code",
      "Functions in the lessons", "Speedup math", "Script defaults".
[AV]  "Adaptive Verification ohne Confidence Head" (spke.com, German) and its
      Arabic mirror "التحقق التكيفي بدون رأس ثقة", sections "Solution: online
      acceptance estimator", "Scoring the distribution", "Other features
      considered", "Fitting the coefficients", footnote 1.

Letters: ``pd`` is the draft distribution and ``pt`` the target distribution.
[CS] names the draft's probabilities p and the verifier's q; [AV] names the
draft q and the target p.  This package never uses bare p or q.

Parity status: every function is pinned by ``tests/test_oracle_*.py`` except
the conventions listed as "parity unpinned" in ``oracle.verify`` and
``oracle.av`` (clamp of the feature at 80, the Z = 0 residual fallback, the
damping constant and ridge values, the T = 0 feature temperature).
"""
from .verify import (  # noqa: F401
    decode_rows,
    log_softmax,
    accept_decision,
    inverse_cdf,
    verify_request,
    verify_batch,
    VerifyResult,
)
from .av import (  # noqa: F401
    feature,
    score,
    survival_and_kept,
    av_score_batch,
    fit_sums,
    newton_step,
    fit_step,
    nll,
)
