"""Oracle of the test-time-speculation distillation gradient - TEST
INFRASTRUCTURE ONLY.

Follows the page "ملخص تقني: التخمين في وقت الاختبار (TTS)" (technical
summary: test-time speculation), section "Algorithm", step 3: before the next
round the draft model takes one gradient step on
    L_t(q) = KL~(p || q) + lambda * KL~(q_t || q),
p the target distribution, q the draft distribution being trained, q_t the
draft distribution that produced the canvas; the first term approximates the
KL divergence between the target and the new draft over the canvas, the
second keeps the draft near its previous state, and position weights w_k
favour early canvas tokens.

Readings (the page gives no formula for the approximation or the weights):

* KL~ over the canvas = sum over canvas positions k of w_k * KL(. || .) of the
  full-vocabulary distributions at that position; the canvas of request b is
  its draft positions k < K_b, the teacher rows are the target rows at the
  same positions;
* every distribution is softmax(logits / T) at the request's temperature T
  (T = 0 counts as T = 1);
* the output is the gradient with respect to the draft logits z of each
  canvas row: w_k * ((q - p) + lambda * (q - q_t)) / T, and the per-position
  loss w_k * (KL(p || q) + lambda * KL(q_t || q)) in nats; when q_t's rows
  are q's own rows the second terms vanish;
* the weights w_k are inputs (parity unpinned: the page gives none).
"""
from __future__ import annotations

import numpy as np


def _softmax(z, T):
    s = np.asarray(z, dtype=np.float64) / T
    s = s - s.max()
    e = np.exp(s)
    return e / e.sum(), s - np.log(e.sum())  # probabilities, log-probabilities


def _kl(logp, logq):
    """sum_v p(v) (log p(v) - log q(v)), terms with p(v) = 0 being 0."""
    p = np.exp(logp)
    live = p > 0
    return float(np.sum(p[live] * (logp[live] - logq[live])))


def position(z_draft, z_target, z_prev, T, w, lam):
    """Gradient row (fp64 [V]) and loss of one canvas position."""
    T = 1.0 if T == 0.0 else float(T)
    q, logq = _softmax(z_draft, T)
    p, logp = _softmax(z_target, T)
    if z_prev is None:
        qt, logqt = q, logq
    else:
        qt, logqt = _softmax(z_prev, T)
    grad = w * ((q - p) + lam * (q - qt)) / T
    loss = w * (_kl(logp, logq) + lam * _kl(logqt, logq))
    return grad, loss
