"""Seeded synthetic verification batches.

Every request draws from its own PCG64 stream (child ``b`` of
``SeedSequence(seed)``), so a batch is independent of how it is chunked or
parallelised and the first ``n`` requests of a batch are the same whatever its
size.  Per request the draws are made in this order: the ragged draft length
(where the workload has one), the draft and target logit rows, the draft
tokens, then the uniforms ``u_accept[max_k]``, ``u_residual`` and ``u_bonus``.

Draft tokens are drawn from the draft distribution at the request's
temperature by the Gumbel-max rule (argmax of logit/T minus the log of a unit
exponential), applied to the stored (bf16-rounded where the workload is bf16)
logits, so that no softmax is computed here.  A greedy request (T = 0) drafts
the lowest-index argmax.

Workloads (logit recipes follow the configurations the verification kernel
is measured on; the speculative-decoding pages give the sizes and acceptance
levels, not these distributions):

``tiny_fp32_b4_k4_v1024``
    B=4, K=4, V=1024, fp32, T=1.  Draft rows ~ N(0, 3^2); target row i =
    draft row i + N(0, 1).  The bonus target row K is built the same way from
    a fresh draft-like row.  Estimator parameters omega=1, beta_i=0.
``bf16_b64_k5_v32000``
    B=64, K=5, V=32000, bf16, T=1.  Draft ~ N(0, 2.5^2); target = 0.9*draft
    + N(0, 1.2^2).  Planted estimator parameters omega=1.2,
    beta_i = 0.5 - 0.3*i.
``bf16_b256_k4_v128256_peaked``
    B=256, K=4, V=128256, bf16, T=1.  Every row is N(0, 2^2) noise plus +6 on
    one token.  The target row shares the draft row's boosted token with
    probability 0.8, else boosts a uniformly chosen different token; its
    noise is independent.  The bonus row boosts a fresh uniform token.
``bf16_b512_k8_v151936_t0.7``
    B=512, K=8, V=151936, bf16, T=0.7.  Draft ~ N(0, 3^2); target = draft +
    N(0, 1.5^2).  Estimator starts at omega=1, beta_i=0; pruning threshold
    0.3 on the cumulative predicted acceptance.
``fp32_b1024_k1to3_v129280_greedy_mix``
    B=1024, K_b uniform on {1,2,3}, V=129280, fp32, packed (ragged) rows.
    Even requests are greedy (T=0), odd ones use T=1.  Each row is N(0, 1)
    with its top token lifted to (runner-up + U(2, 10)); the target's top
    token equals the draft's with probability 0.8.

Filtered-sampling workloads (per-request ``top_k`` / ``top_p`` sampling
parameters; the acceptance-estimator page samples at temperature 1 with
top-p 0.95).  Their draws are those of the workload with the same seed index;
draft tokens are still drawn from the unfiltered draft distribution, so a
draft can fall outside its row's filtered set:

``bf16_b256_k4_v128256_peaked_topp95``
    the peaked B=256, K=4, V=128256 bf16 batch, every request at top-p 0.95.
``bf16_b64_k5_v32000_filter_mix``
    the B=64, K=5, V=32000 bf16 batch with request b unfiltered (b % 4 = 0),
    top-p 0.9 (1), top-k 50 (2), or top-k 200 with top-p 0.8 (3).
``fp32_b32_k4_v1024_filter_mix``
    the tiny recipe (fp32, V=1024) for 32 requests, ragged K_b in 1..4,
    temperatures cycling 1, 0.7, 0 (greedy), 1.3, and the filter settings of
    the previous workload cycling with period 5 (top-k 1, top-k 7, top-p 0.5,
    top-p 0.97 with top-k 600, none).

Logits are generated in fp32 and, for bf16 workloads, rounded to bf16 with
round-to-nearest-even; arrays hold the raw bf16 bit patterns as uint16.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field, replace
from typing import Callable, Optional

import numpy as np


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN logits are not generated")
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# batch container
# --------------------------------------------------------------------------

@dataclass
class Batch:
    """One verification call's worth of host inputs.

    ``draft`` / ``target`` are row-major ``[rows, V]`` arrays: float32, or
    uint16 holding bf16 bits.  Request ``b``'s draft row ``i`` is row
    ``draft_row_start[b] + i`` and its target row ``j`` (0..K_b) is row
    ``target_row_start[b] + j``.
    """

    name: str
    B: int
    V: int
    max_k: int
    dtype: str  # "f32" | "bf16"
    draft: np.ndarray
    draft_row_start: np.ndarray  # int64 [B]
    target: np.ndarray
    target_row_start: np.ndarray  # int64 [B]
    num_draft: np.ndarray  # int32 [B]
    draft_tokens: np.ndarray  # int32 [B, max_k]; unused slots hold 0
    temperature: np.ndarray  # float32 [B]
    u_accept: np.ndarray  # float32 [B, max_k]
    u_residual: np.ndarray  # float32 [B]
    u_bonus: np.ndarray  # float32 [B]
    av_params: np.ndarray  # float32 [max_k + 1] = omega, beta_0..beta_{max_k-1}
    prune_threshold: float = 0.0
    meta: dict = field(default_factory=dict)
    top_k: Optional[np.ndarray] = None  # int32 [B] sampling top-k per request (0: off)
    top_p: Optional[np.ndarray] = None  # float32 [B] sampling top-p per request (1: off)

    def __post_init__(self):
        if self.top_k is None:
            self.top_k = np.zeros(self.B, dtype=np.int32)
        if self.top_p is None:
            self.top_p = np.ones(self.B, dtype=np.float32)

    @property
    def positions(self) -> int:
        """Submitted draft positions: sum of K_b."""
        return int(self.num_draft.sum())

    def rows_f32(self, which: str) -> np.ndarray:
        a = self.draft if which == "draft" else self.target
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a

    def algorithmic_bytes(self, skip_greedy_draft: bool = True) -> int:
        """Bytes of logits a verification call must read once: every
        submitted position's draft row and target row plus each request's
        bonus row.  Greedy requests never need their draft rows."""
        esize = 2 if self.dtype == "bf16" else 4
        k = self.num_draft.astype(np.int64)
        greedy = self.temperature == 0
        draft_rows = np.where(greedy & skip_greedy_draft, 0, k).sum()
        target_rows = (k + 1).sum()
        return int((draft_rows + target_rows) * self.V * esize)


# --------------------------------------------------------------------------
# per-request logit recipes: (rng, K_b, V) -> (draft [K_b,V], target [K_b+1,V]) fp32
# --------------------------------------------------------------------------

def _recipe_tiny(g, k, V):
    d = (3.0 * g.standard_normal((k + 1, V), dtype=np.float32))
    t = d + g.standard_normal((k + 1, V), dtype=np.float32)
    return d[:k], t


def _recipe_llama2(g, k, V):
    d = (2.5 * g.standard_normal((k + 1, V), dtype=np.float32))
    t = 0.9 * d + 1.2 * g.standard_normal((k + 1, V), dtype=np.float32)
    return d[:k], t.astype(np.float32)


def _recipe_peaked(g, k, V):
    d = 2.0 * g.standard_normal((k, V), dtype=np.float32)
    t = 2.0 * g.standard_normal((k + 1, V), dtype=np.float32)
    top_d = g.integers(0, V, size=k)
    share = g.random(k) < 0.8
    other = g.integers(0, V - 1, size=k)
    other = other + (other >= top_d)
    top_t = np.where(share, top_d, other)
    bonus_top = g.integers(0, V)
    d[np.arange(k), top_d] += 6.0
    t[np.arange(k), top_t] += 6.0
    t[k, bonus_top] += 6.0
    return d, t


def _recipe_long(g, k, V):
    d = (3.0 * g.standard_normal((k + 1, V), dtype=np.float32))
    t = d + 1.5 * g.standard_normal((k + 1, V), dtype=np.float32)
    return d[:k], t.astype(np.float32)


def _lift_top(g, rows, top):
    """Set rows[r, top[r]] to the row's runner-up plus a U(2, 10) margin."""
    for r in range(rows.shape[0]):
        rows[r, top[r]] = -np.inf
        rows[r, top[r]] = rows[r].max() + np.float32(g.uniform(2.0, 10.0))


def _recipe_margin(g, k, V):
    d = g.standard_normal((k, V), dtype=np.float32)
    t = g.standard_normal((k + 1, V), dtype=np.float32)
    top_d = g.integers(0, V, size=k)
    share = g.random(k + 1) < 0.8
    other = g.integers(0, V - 1, size=k + 1)
    base = np.concatenate([top_d, g.integers(0, V, size=1)])
    other = other + (other >= base)
    top_t = np.where(share, base, other)
    _lift_top(g, d, top_d)
    _lift_top(g, t, top_t)
    return d, t


@dataclass(frozen=True)
class Workload:
    name: str
    index: int  # seeds are 1000*index + trial
    B: int
    V: int
    max_k: int
    dtype: str
    recipe: Callable
    temperature: Callable  # b -> float
    ragged: bool = False
    omega: float = 1.0
    beta: Callable = lambda i: 0.0
    prune_threshold: float = 0.0
    top_k: Callable = lambda b: 0  # b -> top-k of request b (0: off)
    top_p: Callable = lambda b: 1.0  # b -> top-p of request b (1: off)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32_b4_k4_v1024", 1, 4, 1024, 4, "f32", _recipe_tiny, lambda b: 1.0),
        Workload("bf16_b64_k5_v32000", 2, 64, 32000, 5, "bf16", _recipe_llama2, lambda b: 1.0,
                 omega=1.2, beta=lambda i: 0.5 - 0.3 * i),
        Workload("bf16_b256_k4_v128256_peaked", 3, 256, 128256, 4, "bf16", _recipe_peaked,
                 lambda b: 1.0),
        Workload("bf16_b512_k8_v151936_t0.7", 4, 512, 151936, 8, "bf16", _recipe_long,
                 lambda b: 0.7, prune_threshold=0.3),
        Workload("fp32_b1024_k1to3_v129280_greedy_mix", 5, 1024, 129280, 3, "f32", _recipe_margin,
                 lambda b: 0.0 if b % 2 == 0 else 1.0, ragged=True),
        Workload("bf16_b256_k4_v128256_peaked_topp95", 3, 256, 128256, 4, "bf16", _recipe_peaked,
                 lambda b: 1.0, top_p=lambda b: 0.95),
        Workload("bf16_b64_k5_v32000_filter_mix", 2, 64, 32000, 5, "bf16", _recipe_llama2, lambda b: 1.0,
                 omega=1.2, beta=lambda i: 0.5 - 0.3 * i, top_k=lambda b: (0, 0, 50, 200)[b % 4],
                 top_p=lambda b: (1.0, 0.9, 1.0, 0.8)[b % 4]),
        Workload("fp32_b32_k4_v1024_filter_mix", 1, 32, 1024, 4, "f32", _recipe_tiny,
                 lambda b: (1.0, 0.7, 0.0, 1.3)[b % 4], ragged=True, top_k=lambda b: (1, 7, 0, 600, 0)[b % 5],
                 top_p=lambda b: (1.0, 1.0, 0.5, 0.97, 1.0)[b % 5]),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------

def _gumbel_argmax(g, rows_f32: np.ndarray, T: float) -> np.ndarray:
    """One draw per row from softmax(row / T) by the Gumbel-max rule."""
    z = rows_f32.astype(np.float64)
    if T == 0.0:
        return np.argmax(z, axis=1).astype(np.int32)
    e = g.standard_exponential(z.shape)
    return np.argmax(z / T - np.log(e), axis=1).astype(np.int32)


def _one_request(args):
    name, seed_seq, b, max_k = args
    wl = WORKLOADS[name]
    g = np.random.Generator(np.random.PCG64(seed_seq))
    k = int(g.integers(1, max_k + 1)) if wl.ragged else max_k
    d32, t32 = wl.recipe(g, k, wl.V)
    if wl.dtype == "bf16":
        d_store, t_store = f32_to_bf16_bits(d32), f32_to_bf16_bits(t32)
        d_seen = bf16_bits_to_f32(d_store)
    else:
        d_store, t_store = d32.astype(np.float32), t32.astype(np.float32)
        d_seen = d_store
    T = float(wl.temperature(b))
    toks = _gumbel_argmax(g, d_seen, T) if k > 0 else np.zeros(0, np.int32)
    u_acc = g.random(max_k, dtype=np.float32)
    u_res = g.random(dtype=np.float32)
    u_bon = g.random(dtype=np.float32)
    return k, d_store, t_store, toks, T, u_acc, u_res, u_bon


def make_batch(name: str, trial: int = 0, B: Optional[int] = None, workers: Optional[int] = None) -> Batch:
    """Draw workload ``name`` with seed ``1000*index + trial``.

    ``B`` truncates the batch to its first ``B`` requests (identical to those
    of the full batch).  ``workers`` > 1 draws requests in a thread pool.
    """
    wl = WORKLOADS[name]
    B = wl.B if B is None else int(B)
    seed = 1000 * wl.index + trial
    children = np.random.SeedSequence(seed).spawn(B)
    jobs = [(name, children[b], b, wl.max_k) for b in range(B)]
    big = B * (2 * wl.max_k + 1) * wl.V > 50_000_000
    if workers is None:
        workers = min(8, len(os.sched_getaffinity(0))) if big else 1
    if workers > 1:
        # threads, not processes: numpy's random fills and ufuncs release the
        # GIL, and a thread pool is safe in a process that already holds a GPU
        # context or profiler threads (no fork) and needs no __main__ guard
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(workers) as pool:
            res = list(pool.map(_one_request, jobs))
    else:
        res = [_one_request(j) for j in jobs]

    V, max_k = wl.V, wl.max_k
    ks = np.array([r[0] for r in res], dtype=np.int32)
    if wl.ragged:
        d_start = np.concatenate([[0], np.cumsum(ks)[:-1]]).astype(np.int64)
        t_start = np.concatenate([[0], np.cumsum(ks + 1)[:-1]]).astype(np.int64)
        nd, nt = int(ks.sum()), int((ks + 1).sum())
    else:
        d_start = (np.arange(B, dtype=np.int64) * max_k)
        t_start = (np.arange(B, dtype=np.int64) * (max_k + 1))
        nd, nt = B * max_k, B * (max_k + 1)
    sdt = np.uint16 if wl.dtype == "bf16" else np.float32
    draft = np.zeros((max(nd, 1), V), dtype=sdt)
    target = np.zeros((nt, V), dtype=sdt)
    toks = np.zeros((B, max_k), dtype=np.int32)
    temp = np.zeros(B, dtype=np.float32)
    u_acc = np.zeros((B, max_k), dtype=np.float32)
    u_res = np.zeros(B, dtype=np.float32)
    u_bon = np.zeros(B, dtype=np.float32)
    for b, (k, ds, ts, tk, T, ua, ur, ub) in enumerate(res):
        draft[d_start[b]:d_start[b] + k] = ds
        target[t_start[b]:t_start[b] + k + 1] = ts
        toks[b, :k] = tk
        temp[b], u_acc[b], u_res[b], u_bon[b] = T, ua, ur, ub
    params = np.array([wl.omega] + [wl.beta(i) for i in range(max_k)], dtype=np.float32)
    tk = np.array([wl.top_k(b) for b in range(B)], dtype=np.int32)
    tp = np.array([wl.top_p(b) for b in range(B)], dtype=np.float32)
    return Batch(name, B, V, max_k, wl.dtype, draft, d_start, target, t_start, ks, toks, temp,
                 u_acc, u_res, u_bon, params, wl.prune_threshold, meta={"seed": seed}, top_k=tk, top_p=tp)


# --------------------------------------------------------------------------
# Monte-Carlo sources: fixed rows shared by every request (row starts all 0)
# --------------------------------------------------------------------------

def constant_alpha_rows(alpha: float, V: int, K: int, seed: int):
    """Draft/target probability rows whose per-position overlap is exactly
    ``alpha``: with w a random full-support distribution (normalised unit
    exponentials), draft = alpha*w + (1-alpha)*onehot(0) and target =
    alpha*w + (1-alpha)*onehot(1).  Returns (pd [K, V], pt [K+1, V]) in fp64."""
    g = np.random.Generator(np.random.PCG64(seed))
    pd = np.empty((K, V))
    pt = np.empty((K + 1, V))
    for i in range(K + 1):
        w = g.standard_exponential(V)
        w /= w.sum()
        if i < K:
            pd[i] = alpha * w
            pd[i, 0] += 1.0 - alpha
        w2 = g.standard_exponential(V)
        w2 /= w2.sum()
        pt[i] = alpha * (w if i < K else w2)
        pt[i, 1] += 1.0 - alpha
    return pd, pt


def broadcast_batch(draft_rows: np.ndarray, target_rows: np.ndarray, trials: int, seed: int,
                    draft_probs: Optional[np.ndarray] = None, temperature: float = 1.0,
                    name: str = "broadcast") -> Batch:
    """``trials`` requests that all read the same K draft rows and K+1 target
    rows (row starts 0), each with fresh draft tokens and uniforms.

    ``draft_rows``/``target_rows`` are fp32 logits.  Tokens are drawn from
    ``draft_probs`` (explicit probabilities) when given, else by Gumbel-max on
    the draft logits at ``temperature``.
    """
    K, V = draft_rows.shape
    g = np.random.Generator(np.random.PCG64(seed))
    toks = np.empty((trials, K), dtype=np.int32)
    for i in range(K):
        if draft_probs is not None:
            p = draft_probs[i] / draft_probs[i].sum()
            toks[:, i] = g.choice(V, size=trials, p=p)
        else:
            z = draft_rows[i].astype(np.float64)
            if temperature == 0.0:
                toks[:, i] = int(np.argmax(z))
            else:
                for s in range(0, trials, 4096):
                    n = min(4096, trials - s)
                    e = g.standard_exponential((n, V))
                    toks[s:s + n, i] = np.argmax(z[None, :] / temperature - np.log(e), axis=1)
    u_acc = g.random((trials, K), dtype=np.float32)
    u_res = g.random(trials, dtype=np.float32)
    u_bon = g.random(trials, dtype=np.float32)
    zeros = np.zeros(trials, dtype=np.int64)
    return Batch(name, trials, V, K, "f32", np.ascontiguousarray(draft_rows, dtype=np.float32), zeros,
                 np.ascontiguousarray(target_rows, dtype=np.float32), zeros.copy(),
                 np.full(trials, K, dtype=np.int32), toks, np.full(trials, temperature, np.float32),
                 u_acc, u_res, u_bon, np.array([1.0] + [0.0] * K, dtype=np.float32), 0.0,
                 meta={"seed": seed})


def subset(batch: Batch, idx) -> Batch:
    """Requests ``idx`` of ``batch`` (row arrays shared, starts kept)."""
    idx = np.asarray(idx)
    return replace(batch, B=len(idx), draft_row_start=batch.draft_row_start[idx],
                   target_row_start=batch.target_row_start[idx], num_draft=batch.num_draft[idx],
                   draft_tokens=batch.draft_tokens[idx], temperature=batch.temperature[idx],
                   u_accept=batch.u_accept[idx], u_residual=batch.u_residual[idx],
                   u_bonus=batch.u_bonus[idx], top_k=batch.top_k[idx], top_p=batch.top_p[idx])
