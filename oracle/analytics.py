"""Oracle for acceptance analytics of one verification step.

TEST INFRASTRUCTURE ONLY (see the package docstring). Written from "Speculative decoding:
accelerate LLM generation without changing its answers":

* section 3 "Why this preserves the target distribution": at one position a proposal x
  drawn from q is accepted with probability min(1, p(x)/q(x)), so the accepted mass is
  min(q, p) token by token and the probability that the position accepts is
  beta = sum_x min(p(x), q(x)); the residual total sum_x max(0, p(x) - q(x)) is the
  probability of rejection, 1 - beta (the toy lab of section 5 prints 0.3 for it).
* section 4 "Data flow and performance trade-offs": E[A], the expected output of a cycle
  counting the correction or bonus token, enters the throughput proxy E[A] / (D(k) + V(k)).

Reading (the pages give E[A] without a formula): with the proposal rows of a cycle fixed
(p_i, q_i at positions i = 1..k for the drafted prefix) and each y_i drawn from q_i, the
cycle emits at least j + 1 tokens iff positions 1..j all accept, with probability
beta_1 * ... * beta_j; so E[A] = 1 + sum_{j=1..k} prod_{i<=j} beta_i.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .verify import _decode_rows, params_ok, transform


def acceptance_rate(p, q):
    """beta = sum_x min(p(x), q(x)): the probability that a proposal drawn from q is
    accepted at this position (floats, NumPy arrays or Fractions)."""
    if isinstance(p, np.ndarray):
        return float(np.minimum(p, q).sum())
    total = 0 * p[0]
    for pi, qi in zip(p, q):
        total = total + min(pi, qi)
    return total


def expected_emitted(betas: Sequence):
    """E[A] = 1 + sum_j prod_{i<=j} beta_i (the correction or bonus token included)."""
    e = 1 + 0 * (betas[0] if len(betas) else 0)
    run = 1 + 0 * e
    for b in betas:
        run = run * b
        e = e + run
    return e


def acceptance_batch(target, draft, cu_draft, T, top_k, dtype: str, top_p=1.0,
                     top_k_max=None, requests: Optional[Sequence[int]] = None,
                     draft_tokens=None, u_accept=None, u_sample=None):
    """Per-position beta_i [K] and per-request E[A] [B] of a packed ragged batch (rows as
    in verify_batch). Requests that fail verification get NaN: malformed offsets, invalid
    parameters, a row that cannot be normalized and, when the proposals and uniforms are
    given, a token outside [0, V) or a uniform outside [0, 1)."""
    cu = np.asarray(cu_draft, dtype=np.int64)
    B = cu.shape[0] - 1
    K = int(draft.shape[0])
    V = int(target.shape[1])
    per = lambda x, f: [f(v) for v in np.broadcast_to(np.asarray(x), (B,))]
    Ts = per(T, lambda v: float(np.float32(v)))
    ks = per(top_k, int)
    ps = per(top_p, lambda v: float(np.float32(v)))
    beta = np.full(K, np.nan)
    E = np.full(B, np.nan)
    bad_cu = cu[0] != 0 or cu[B] != K or np.any(np.diff(cu) < 0)
    for b in (range(B) if requests is None else requests):
        if bad_cu:
            continue
        lo, hi = int(cu[b]), int(cu[b + 1])
        if not params_ok(Ts[b], ks[b], ps[b], V, top_k_max):
            continue
        if draft_tokens is not None and any(not 0 <= int(y) < V for y in draft_tokens[lo:hi]):
            continue
        if u_accept is not None and not all(0.0 <= float(u) < 1.0
                                            for u in list(u_accept[lo:hi]) + [u_sample[b]]):
            continue
        t_rows = _decode_rows(target[lo + b: hi + b + 1], dtype)
        d_rows = _decode_rows(draft[lo:hi], dtype)
        rows_t = [transform(t_rows[i], Ts[b], ks[b], ps[b]) for i in range(hi - lo + 1)]
        rows_d = [transform(d_rows[i], Ts[b], ks[b], ps[b]) for i in range(hi - lo)]
        if not all(r.valid for r in rows_t + rows_d):
            continue
        betas: List[float] = [acceptance_rate(rows_t[i].p, rows_d[i].p) for i in range(hi - lo)]
        beta[lo:hi] = betas
        E[b] = expected_emitted(betas)
    return beta, E
