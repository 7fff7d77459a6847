"""Statistical checks of the GPU path: emitted tokens follow the target
distribution (chi-square, the cheat sheet's `chi_square(observed, expected)`
check) and the accept length on a constant-alpha source matches the
tokens-per-verify closed form.  All trials read the same rows (row starts 0)
with fresh draft tokens and uniforms, so one launch runs many trials."""
import numpy as np
import pytest
import scipy.special as sp
import scipy.stats as st
import torch

from conftest import load_golden
from gpu_harness import gpu_verify
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]


def chi_square_p(observed, expected_probs, min_expected=5.0):
    observed = np.asarray(observed, np.float64)
    exp = np.asarray(expected_probs, np.float64) * observed.sum()
    o_m, e_m, ao, ae = [], [], 0.0, 0.0
    for i in np.argsort(exp):
        ao += observed[i]
        ae += exp[i]
        if ae >= min_expected:
            o_m.append(ao)
            e_m.append(ae)
            ao = ae = 0.0
    if ae > 0:
        o_m[-1] += ao
        e_m[-1] += ae
    return st.chisquare(o_m, e_m).pvalue


@pytest.mark.parametrize("V,seed", [(8, 0), (1024, 1)])
def test_emitted_tokens_follow_target(V, seed):
    K, M = 4, 200_000
    g = np.random.default_rng(seed)
    scale = 1.5 if V == 8 else 3.0
    zd = (scale * g.standard_normal((K, V))).astype(np.float32)
    zt = np.vstack([zd + g.standard_normal((K, V)), scale * g.standard_normal((1, V)) + g.standard_normal((1, V))])
    zt = zt.astype(np.float32)
    pd = np.stack([sp.softmax(zd[i].astype(np.float64)) for i in range(K)])
    b = gen.broadcast_batch(zd, zt, M, seed=seed + 10, draft_probs=pd)
    print(f"case chi-square V={V} M={M}", flush=True)
    out = gpu_verify(b)
    toks = out["out_tokens"]
    for j in range(K + 1):
        reached = toks[:, j] >= 0
        if reached.sum() < 1000:
            continue
        counts = np.bincount(toks[reached, j], minlength=V)
        p = chi_square_p(counts, sp.softmax(zt[j].astype(np.float64)))
        assert p > 1e-4, (j, p, reached.sum())


@pytest.mark.parametrize("which", ["golden", "command"])
def test_accept_length_matches_closed_form(which):
    if which == "golden":
        gd = load_golden("tokens_per_verify.txt")
        alpha, K, V, M = gd["alpha"], int(gd["K"]), 64, 1_000_000
    else:  # the demo command line: vocab 64, alpha 0.75, k 4, 50000 samples
        sd = load_golden("script_defaults.txt")
        alpha, K, V, M = sd["alpha"], int(sd["k"]), int(sd["command_vocab"]), int(sd["command_samples"])
    pd, pt = gen.constant_alpha_rows(alpha, V=V, K=K, seed=3)
    b = gen.broadcast_batch(np.log(pd).astype(np.float32), np.log(pt).astype(np.float32), M, seed=4,
                            draft_probs=pd)
    print(f"case constant alpha={alpha} K={K} V={V} M={M}", flush=True)
    parts = [gpu_verify(gen.subset(b, np.arange(s, min(M, s + 200_000)))) for s in range(0, M, 200_000)]
    out = {k: np.concatenate([p_[k] for p_ in parts]) for k in parts[0]}
    n = out["accept_len"].astype(np.float64) + 1
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    se = n.std(ddof=1) / np.sqrt(M)
    assert abs(n.mean() - closed) < 4 * se, (n.mean(), closed, se)
    if which == "golden":
        assert abs(n.mean() - gd["tokens_per_verify"]) < 0.005 + 4 * se
    hist = np.bincount(out["accept_len"], minlength=K + 1)
    probs = [alpha ** j * (1 - alpha) for j in range(K)] + [alpha ** K]
    assert chi_square_p(hist, probs) > 1e-4
