"""Oracle for the verification step: transform, accept test, residual / bonus sampling.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain fp64 NumPy, or exact
``fractions.Fraction`` arithmetic through the generic functions, following the pages in
their own order and notation. Nothing here is blocked, fused or reordered.

Method, from "Speculative decoding: accelerate LLM generation without changing its
answers", section 2 "Draft, verify, correct":

* p_i is the target distribution and q_i the draft distribution at proposal position i,
  both after the same decoding transform (section 3 closing paragraph and section 6,
  "Distribution mismatch").
* Each proposal y_i is accepted with probability min(1, p_i(y_i) / q_i(y_i)), left to
  right; the first rejection ends the run and later proposals are discarded.
* At the first rejection a replacement is drawn from normalize(max(0, p_i - q_i)).
* If every proposal is accepted, one bonus token is drawn from the target distribution
  after the block (p_{k+1}).

Readings taken where the pages leave a step open (each is listed in the design notes):

* accept iff ``u * Q < P`` with u uniform on [0, 1). This has probability min(1, P/Q),
  accepts whenever P >= Q, rejects when P = 0, and never divides by Q (section 5,
  variation 2 asks that p/q is not evaluated at q = 0).
* inverse CDF walks token ids in ascending order and returns the smallest x whose running
  sum C(x) exceeds t = u * W, with W the final running sum. If rounding leaves no such x,
  the last x with positive weight is taken.
* a residual mass of 0 after a rejection cannot happen in exact arithmetic when the
  proposal was drawn from q_i (section 3: the rejection probability equals the residual
  mass), but it can when the two distributions agree and the proposal lies outside both
  (a transform dropped it). Then the replacement is drawn from p_i and the request is
  flagged (section 6: never divide by zero). Zero is decided on the fp64 sum: p and q
  that agree exactly (equal kept sets, logits equal up to one common shift) are computed
  by the same fp64 operations on the same values z - m and are bitwise equal, so their
  residual sums to exactly 0; any other pair leaves a positive fp64 residual.
* top-k keeps every token whose logit is >= the k-th largest logit of the row, counting
  multiplicity (ties inclusive), and selects on the raw logits, which is the same set for
  any temperature T > 0.
* top-p (the pages name it among the transforms that must be applied identically to both
  distributions, section 3 closing paragraph and section 4, without defining it) is the
  nucleus rule, applied after temperature and top-k to the renormalized kept
  distribution: keep every token whose probability is >= the largest value v for which
  the tokens with probability >= v carry at least top_p of the mass (ties inclusive, like
  top-k); top_p <= 0 or >= 1 leaves the row unchanged.
* the bonus token is emitted only when all proposals are accepted (section 2, section 6
  "Bad bonus-token logic").
* stopping ("Keep cache validity aligned with the committed token history", paragraph 6
  names EOS and output caps among the cases to test): a request's output ends at the first
  accepted proposal equal to its end-of-sequence token (inclusive), or after its cap of
  tokens, when that falls within the accepted proposals; then nothing is drawn and the
  accepted count is the number of tokens kept (the cache keeps their states). A drawn
  replacement or bonus equal to EOS ends the output naturally.
* temperature, top-k and top-p may differ between the requests of a batch; within a
  request the same values shape every p_i and q_i. A request whose temperature is not
  a positive finite number, whose top_p is NaN, or whose active top_k exceeds the
  caller's declared bound fails (ERR_PARAM) and samples nothing.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# Per-request error / flag bits of the verification step. Error bits make the request's
# outputs invalid (num_accepted = -1, num_emitted = 0); flag bits are informational.
ERR_TOKEN = 1          # a draft token id outside [0, V)
ERR_K = 2              # ragged offsets inconsistent: k_b < 0, k_b > max_k, cu[0] != 0, cu[B] != K
ERR_NONFINITE = 4      # NaN or +inf logit in a row, or a row with no finite kept logit
ERR_QZERO = 8          # flag: q_i(y_i) == 0 at an evaluated position
ERR_ZFALLBACK = 16     # flag: residual mass 0 after a rejection; drew from p_i instead
ERR_UNIFORM = 32       # a caller uniform outside [0, 1) or NaN
ERR_PARAM = 64         # the request's temperature / top_p / top_k is invalid

ERROR_BITS = ERR_TOKEN | ERR_K | ERR_NONFINITE | ERR_UNIFORM | ERR_PARAM


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# Decoding transform (temperature, optional top-k), applied identically to p and q.
# --------------------------------------------------------------------------------------

@dataclass
class Transformed:
    """One row after the decoding transform."""
    p: Optional[np.ndarray]   # normalized probabilities, float64 [V]; None if invalid
    m: float                  # max kept logit
    S: float                  # sum over kept x of exp((z(x) - m) / T)
    thr: float                # smallest kept logit under top-k / top-p (-inf when both are off)
    nkept: int                # number of kept tokens with finite logit
    valid: bool
    # top-p: distance of the nucleus mass decision from top_p (the mass through the
    # boundary value minus top_p, and top_p minus the mass above it), inf when off
    nucleus_margin: float = math.inf


def transform(z: np.ndarray, T: float, top_k: int, top_p: float = 1.0) -> Transformed:
    """Temperature + top-k + top-p transform of one logit row, stable softmax in fp64.

    Section 6 of the speculative-decoding lesson asks for stable softmax and for the same
    transform on both distributions; section 4 ("When it wins") lists temperature and
    top-k among the transforms that shape p and q. Softmax is max-subtracted.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if np.isnan(z).any() or np.isposinf(z).any():
        return Transformed(None, math.nan, math.nan, math.nan, 0, False)
    if 0 < top_k < V:
        # k-th largest value counting multiplicity
        thr = float(np.partition(z, V - top_k)[V - top_k])
    else:
        thr = -math.inf
    kept = (z >= thr) & (z > -math.inf)
    nkept = int(kept.sum())
    if nkept == 0:
        return Transformed(None, -math.inf, 0.0, thr, 0, False)
    m = float(z[kept].max())
    with np.errstate(invalid="ignore", over="ignore"):
        e = np.where(kept, np.exp((z - m) / T), 0.0)
    S = float(e.sum())
    margin = math.inf
    if 0.0 < top_p < 1.0:
        thr, margin = nucleus(z[kept], e[kept] / S, top_p)
        kept = (z >= thr) & (z > -math.inf)
        nkept = int(kept.sum())
        e = np.where(kept, e, 0.0)
        S = float(e.sum())
    return Transformed(e / S, m, S, thr, nkept, True, margin)


def nucleus(zk: np.ndarray, pk: np.ndarray, top_p: float):
    """Smallest kept logit of the nucleus and the margin of its mass decision.

    zk, pk: logits and normalized probabilities of the kept tokens. Equal logits have equal
    probability, so the values are walked in descending order, one group of equal values
    at a time, until the mass of the groups taken reaches top_p."""
    vals = np.unique(zk)[::-1]                 # distinct kept logits, descending
    before = 0.0
    for v in vals:
        through = before + float(pk[zk == v].sum())
        if through >= top_p:
            return float(v), min(through - top_p, top_p - before)
        before = through
    # rounding left the total short of top_p: keep every kept token
    return float(vals[-1]), 0.0


# --------------------------------------------------------------------------------------
# Generic (works on floats and on fractions.Fraction) accept / residual / inverse CDF.
# --------------------------------------------------------------------------------------

def accept(P, Q, u) -> bool:
    """Accept the proposal iff u * Q < P (probability min(1, P/Q) for u ~ U[0, 1))."""
    return u * Q < P


def residual_weights(p, q):
    """Unnormalized residual max(0, p(x) - q(x)) per token (lesson section 2 and 3)."""
    if isinstance(p, np.ndarray):
        return np.maximum(p - q, 0.0)
    return [max(pi - qi, 0 * pi) for pi, qi in zip(p, q)]


def inverse_cdf(w: Sequence, u):
    """Smallest x (ascending id) with running sum C(x) > u * W, W = final running sum.

    Returns (x, W, margin) where margin = min(t - C(x-1), C(x) - t) / W is the distance of
    t = u * W to the nearer edge of x's CDF interval, as a fraction of W. Returns
    (None, W, None) when no weight is positive. Plain loop: meant for small V and exact
    arithmetic; ``inverse_cdf_np`` is the NumPy form for large rows.
    """
    W = 0 * u
    for v in w:
        W = W + v
    if not W > 0:
        return None, W, None
    t = u * W
    C = 0 * u
    for x, v in enumerate(w):
        prev = C
        C = C + v
        if C > t:
            return x, W, min(t - prev, C - t) / W
    last = max(x for x, v in enumerate(w) if v > 0)
    return last, W, 0 * W


def inverse_cdf_np(w: np.ndarray, u: float):
    """``inverse_cdf`` for float64 NumPy rows (sequential cumulative sum, same rule)."""
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    if C.shape[0] == 0 or not C[-1] > 0:
        return None, (float(C[-1]) if C.shape[0] else 0.0), None
    W = float(C[-1])
    t = float(u) * W
    x = int(np.searchsorted(C, t, side="right"))
    if x >= C.shape[0]:
        pos = np.nonzero(np.asarray(w) > 0)[0]
        return int(pos[-1]), W, 0.0
    prev = float(C[x - 1]) if x > 0 else 0.0
    return x, W, min(t - prev, float(C[x]) - t) / W


def _icdf(w, u):
    if isinstance(w, np.ndarray):
        return inverse_cdf_np(w, u)
    return inverse_cdf(w, u)


@dataclass
class ProbsResult:
    a: int                      # accepted proposals
    emitted: List[int]          # y_1..y_a followed by the replacement or bonus token
    P: list                     # p_i(y_i) for every position i < k
    Q: list                     # q_i(y_i)
    accept_margin: list         # |u_i - P_i/Q_i| (inf when Q_i = 0)
    mode: str                   # "resid" or "bonus"
    W: object                   # total weight sampled from (residual mass, or sum p)
    picked: object              # w(x*) / W
    sample_margin: object
    flags: int                  # ERR_QZERO / ERR_ZFALLBACK
    W_resid: object = None      # residual mass before any fallback (None for the bonus)


def verify_probs(P_rows, Q_rows, tokens, u_accept, u_sample) -> ProbsResult:
    """One request's verification on given probability vectors.

    P_rows[0..k] are the target distributions at the k proposal positions plus the one
    after the block; Q_rows[0..k-1] the draft distributions. Generic arithmetic, so exact
    tests can pass Fractions.
    """
    k = len(tokens)
    P, Q, margins = [], [], []
    for i in range(k):
        y = tokens[i]
        P.append(P_rows[i][y])
        Q.append(Q_rows[i][y])
        margins.append(abs(u_accept[i] - P[i] / Q[i]) if Q[i] != 0 else math.inf)
    flags = 0
    a = k
    for i in range(k):
        if Q[i] == 0:
            flags |= ERR_QZERO
        if not accept(P[i], Q[i], u_accept[i]):
            a = i
            break
    if a < k:
        mode = "resid"
        w = residual_weights(P_rows[a], Q_rows[a])
        x, W, margin = _icdf(w, u_sample)
        W_resid = W
        if x is None:
            # the residual has no mass (W == 0): draw from p_i instead
            flags |= ERR_ZFALLBACK
            w = P_rows[a]
            x, W, margin = _icdf(w, u_sample)
    else:
        mode = "bonus"
        W_resid = None
        w = P_rows[k]
        x, W, margin = _icdf(w, u_sample)
    picked = w[x] / W
    emitted = [int(t) for t in tokens[:a]] + [int(x)]
    return ProbsResult(a, emitted, P, Q, margins, mode, W, picked, margin, flags, W_resid)


# --------------------------------------------------------------------------------------
# Logit-level request and batch.
# --------------------------------------------------------------------------------------

@dataclass
class RequestResult:
    a: int                          # -1 on error
    emitted: List[int]
    err: int
    probs: Optional[ProbsResult]
    rows_t: List[Transformed] = field(default_factory=list)
    rows_d: List[Transformed] = field(default_factory=list)


def _u_ok(u) -> bool:
    u = float(u)
    return 0.0 <= u < 1.0


def params_ok(T: float, top_k: int, top_p: float, V: int, top_k_max=None) -> bool:
    """Whether one request's transform parameters are valid."""
    if not (T > 0.0 and math.isfinite(T)) or math.isnan(top_p):
        return False
    return top_k_max is None or not (0 < top_k < V) or top_k <= top_k_max


def verify_request(t_rows, d_rows, tokens, u_accept, u_sample, T: float, top_k: int,
                   V: int, keep_probs: bool = True, top_p: float = 1.0,
                   top_k_max=None) -> RequestResult:
    """Validate and verify one request from logits (float64 rows). With keep_probs=False
    the normalized rows are dropped from the result once used (large vocabularies)."""
    k = len(tokens)
    err = 0
    if any((int(y) < 0 or int(y) >= V) for y in tokens):
        err |= ERR_TOKEN
    if not all(_u_ok(u) for u in u_accept) or not _u_ok(u_sample):
        err |= ERR_UNIFORM
    if not params_ok(T, top_k, top_p, V, top_k_max):
        return RequestResult(-1, [], err | ERR_PARAM, None)
    rows_t = [transform(t_rows[i], T, top_k, top_p) for i in range(k + 1)]
    rows_d = [transform(d_rows[i], T, top_k, top_p) for i in range(k)]
    if not all(r.valid for r in rows_t) or not all(r.valid for r in rows_d):
        err |= ERR_NONFINITE
    if err & ERROR_BITS:
        res = None
    else:
        res = verify_probs([r.p for r in rows_t], [r.p for r in rows_d],
                           [int(y) for y in tokens],
                           [float(u) for u in u_accept], float(u_sample))
    if not keep_probs:
        for r in rows_t + rows_d:
            r.p = None
    if res is None:
        return RequestResult(-1, [], err, None, rows_t, rows_d)
    return RequestResult(res.a, res.emitted, err | res.flags, res, rows_t, rows_d)


def _stop(r: RequestResult, eos, cap) -> RequestResult:
    """Truncate one request's output at its first accepted EOS or at its cap. A cut
    request draws nothing, so the flag that describes the draw (ERR_ZFALLBACK) is dropped;
    ERR_QZERO still reports every evaluated position."""
    L = r.a + 1
    if eos is not None and eos >= 0:
        for i, y in enumerate(r.emitted[:r.a]):
            if y == eos:
                L = i + 1
                break
    if cap is not None and 0 < cap < L:
        L = cap
    if L > r.a:
        return r
    return RequestResult(L, r.emitted[:L], r.err & ~ERR_ZFALLBACK, r.probs, r.rows_t, r.rows_d)


@dataclass
class BatchResult:
    num_accepted: np.ndarray     # int32 [B]
    num_emitted: np.ndarray      # int32 [B]
    out_tokens: np.ndarray       # int32 [K+B], -1 where nothing was emitted
    err: np.ndarray              # int32 [B] per-request bits
    err_word: int                # OR of all bits
    requests: List[Optional[RequestResult]]


def _decode_rows(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def verify_batch(target, draft, draft_tokens, cu_draft, u_accept, u_sample,
                 T, top_k, max_k: int, dtype: str,
                 requests: Optional[Sequence[int]] = None,
                 keep_probs: bool = True, top_p=1.0, top_k_max=None, eos=None,
                 max_emit=None) -> BatchResult:
    """Batched verification over packed ragged rows.

    target: [K+B, V] (fp32 values, or bf16 bit patterns as uint16); the rows of request b
    are cu[b] + b + i for i = 0..k_b. draft: [K, V]; rows cu[b] + i for i < k_b.
    T, top_k, top_p: one value for every request, or one per request (T and top_p are
    rounded to fp32). top_k_max: the bound on active per-request top_k values, if any.
    ``requests`` restricts the work to a subset (other entries stay -1 / 0).
    """
    cu = np.asarray(cu_draft, dtype=np.int64)
    B = cu.shape[0] - 1
    K = int(np.asarray(draft_tokens).shape[0])
    V = int(target.shape[1])
    per = lambda x, f: [f(v) for v in np.broadcast_to(np.asarray(x), (B,))]
    Ts = per(T, lambda v: float(np.float32(v)))
    ks = per(top_k, int)
    ps = per(top_p, lambda v: float(np.float32(v)))
    num_acc = np.full(B, -1, dtype=np.int32)
    num_emit = np.zeros(B, dtype=np.int32)
    out = np.full(K + B, -1, dtype=np.int32)
    errs = np.zeros(B, dtype=np.int32)
    results: List[Optional[RequestResult]] = [None] * B
    bad_cu = (cu[0] != 0) or (cu[B] != K)
    for b in (range(B) if requests is None else requests):
        lo, hi = int(cu[b]), int(cu[b + 1])
        k = hi - lo
        if bad_cu or k < 0 or k > max_k or lo < 0 or hi > K:
            errs[b] = ERR_K
            continue
        t_rows = _decode_rows(target[lo + b: lo + b + k + 1], dtype)
        d_rows = _decode_rows(draft[lo: hi], dtype)
        r = verify_request(t_rows, d_rows, np.asarray(draft_tokens[lo:hi]),
                           np.asarray(u_accept[lo:hi]), u_sample[b], Ts[b], ks[b], V, keep_probs,
                           ps[b], top_k_max)
        if r.a >= 0:
            r = _stop(r, None if eos is None else int(eos[b]),
                      None if max_emit is None else int(max_emit[b]))
        results[b] = r
        errs[b] = r.err
        if r.a >= 0:
            num_acc[b] = r.a
            num_emit[b] = len(r.emitted)
            out[lo + b: lo + b + len(r.emitted)] = r.emitted
    return BatchResult(num_acc, num_emit, out, errs, int(np.bitwise_or.reduce(errs)) if B else 0,
                       results)
