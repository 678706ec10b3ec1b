"""Oracle for verification of a draft tree, and the cache step that keeps the accepted path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix the linear rule ("Speculative decoding: accelerate LLM generation without
changing its answers", section 2: accept y with probability min(1, p(y)/q(y)); at a
rejection draw from normalize(max(0, p - q)); the bonus after a fully accepted block) and
say of trees only what the cache must do ("Keep cache validity aligned with the committed
token history", paragraph 3: a tree implementation gathers the accepted path into the
cache layout and removes the sibling references; paragraph 6 asks for tests of tree
branch switches). Reading taken for the verification of a tree (stated in the design
notes): the children of a node are alternatives for the same next position, each a draw
from that node's draft distribution q. They are tried in node order against a running
target distribution that starts as p and, after each rejected child, becomes the
normalized residual of section 2, normalize(max(0, p' - q)). The first accepted child
continues the walk from its own rows; when every child is rejected the replacement is
drawn from the last residual; a node reached by acceptance that has no children emits the
bonus token from its p. With one child per node this is the linear rule, and applying
section 3's argument at each rejection (the residual carries exactly the target mass not
yet accounted for) keeps the output distributed as the target.

Tree layout: node j of a request (0 <= j < n) has a token and a parent in {-1, 0, .., j-1}
(-1: a child of the root, the position after the committed prefix). Distribution rows are
indexed by position: row 0 the root, row 1 + j the position after node j.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .kv import KV_APPEND_REJECTED, KV_ERR_ROLLBACK, PagedKV
from .verify import (ERR_K, ERR_NONFINITE, ERR_PARAM, ERR_QZERO, ERR_TOKEN, ERR_UNIFORM,
                     ERR_ZFALLBACK, _decode_rows, _icdf, _u_ok, accept, params_ok,
                     residual_weights, transform)

ERR_TREE = 128          # a parent index outside {-1, .., j-1}

ERROR_BITS_TREE = ERR_TOKEN | ERR_K | ERR_NONFINITE | ERR_UNIFORM | ERR_TREE | ERR_PARAM


def children_of(parent: Sequence[int]) -> List[List[int]]:
    """Children of every position (0: root, 1 + j: node j), in node order."""
    kids: List[List[int]] = [[] for _ in range(len(parent) + 1)]
    for j, pa in enumerate(parent):
        kids[int(pa) + 1].append(j)
    return kids


@dataclass
class TreeResult:
    path: List[int]             # accepted nodes, root to deepest
    emitted: List[int]          # their tokens, then the replacement or bonus token
    flags: int
    accept_margin: List[float] = field(default_factory=list)  # |u - P/Q| of every tried node
    sample_margin: float = math.inf
    W: object = None            # total weight of the final draw
    tried: List[int] = field(default_factory=list)             # nodes tested, in order
    resid_W: list = field(default_factory=list)  # residual mass after each rejected child


def tree_verify_probs(P_rows, Q_rows, parent, tokens, u_accept, u_sample,
                      P_of=None, Q_of=None) -> TreeResult:
    """Walk one request's tree on given distributions (generic arithmetic: floats, NumPy
    or Fractions). P_rows[v] / Q_rows[v] for positions v; P_of / Q_of, if given, are
    called with v instead (rows built on demand)."""
    get_p = P_of or (lambda v: P_rows[v])
    get_q = Q_of or (lambda v: Q_rows[v])
    kids = children_of(parent)
    v, path, flags = 0, [], 0
    margins: List[float] = []
    tried: List[int] = []
    resid_W: list = []
    while True:
        p = get_p(v)
        if not kids[v]:
            w = p                                   # bonus from p at a leaf
        else:
            q = get_q(v)
            w = None
            nxt = None
            for j in kids[v]:
                y = int(tokens[j])
                tried.append(j)
                P, Q = p[y], q[y]
                margins.append(abs(u_accept[j] - P / Q) if Q != 0 else math.inf)
                if Q == 0:
                    flags |= ERR_QZERO
                if accept(P, Q, u_accept[j]):
                    nxt = j
                    break
                r = residual_weights(p, q)
                W = sum(r)
                resid_W.append(W)
                if not W > 0:
                    # residual mass 0 (the tested distribution and q agree exactly): the
                    # replacement is drawn from the distribution the child was tested
                    # against
                    flags |= ERR_ZFALLBACK
                    w = p
                    break
                w = r
                p = [x / W for x in r] if not isinstance(r, np.ndarray) else r / W
            if nxt is not None:
                path.append(nxt)
                v = nxt + 1
                continue
        x, W, margin = _icdf(w, u_sample)
        emitted = [int(tokens[j]) for j in path] + [int(x)]
        return TreeResult(path, emitted, flags, margins, margin, W, tried, resid_W)


@dataclass
class TreeRequestResult:
    a: int                      # accepted path length, -1 on error
    path: List[int]
    emitted: List[int]
    err: int
    res: Optional[TreeResult]
    # top-p: the smallest nucleus margin of the rows the walk read (inf when off)
    nucleus_margin: float = math.inf


def tree_verify_request(t_rows, d_rows, parent, tokens, u_accept, u_sample, T: float,
                        V: int, top_k: int = 0, top_p: float = 1.0,
                        top_k_max=None) -> TreeRequestResult:
    """One request from logits (fp64 rows by position); the decoding transform (temperature,
    then top-k, then top-p) applied alike to every target and draft row ("Speculative
    decoding: accelerate LLM generation without changing its answers", section 3's closing
    paragraph and section 4: p and q must come from the same transform), stable softmax,
    rows transformed only where the walk reads them. Invalid parameters (as for the linear
    rule: T not positive and finite, top_p NaN, an active top_k above top_k_max) fail the
    request with ERR_PARAM."""
    n = len(tokens)
    err = 0
    if not params_ok(T, top_k, top_p, V, top_k_max):
        err |= ERR_PARAM
    if any(not (-1 <= int(pa) < j) for j, pa in enumerate(parent)):
        err |= ERR_TREE
    if any(not 0 <= int(y) < V for y in tokens):
        err |= ERR_TOKEN
    if not all(_u_ok(u) for u in u_accept) or not _u_ok(u_sample):
        err |= ERR_UNIFORM
    if err:
        return TreeRequestResult(-1, [], [], err, None)
    cache = {}
    bad = []
    margin = [math.inf]

    def row(which, v):
        key = (which, v)
        if key not in cache:
            t = transform((t_rows if which == 0 else d_rows)[v], T, top_k, top_p)
            margin[0] = min(margin[0], t.nucleus_margin)
            if not t.valid:
                bad.append(v)
                t = None
            cache[key] = t
        t = cache[key]
        if t is None:
            raise _BadRow()
        return t.p

    try:
        res = tree_verify_probs(None, None, parent, tokens, u_accept, u_sample,
                                P_of=lambda v: row(0, v), Q_of=lambda v: row(1, v))
    except _BadRow:
        return TreeRequestResult(-1, [], [], ERR_NONFINITE, None, margin[0])
    return TreeRequestResult(len(res.path), res.path, res.emitted, res.flags, res, margin[0])


class _BadRow(Exception):
    pass


@dataclass
class TreeBatchResult:
    num_accepted: np.ndarray     # [B]
    num_emitted: np.ndarray      # [B]
    out_tokens: np.ndarray       # [N + B]: request b at cu[b] + b
    accepted_nodes: np.ndarray   # [N]: request b's path at cu[b] .. cu[b] + a - 1
    err: np.ndarray              # [B]
    requests: List[Optional[TreeRequestResult]]


def tree_verify_batch(target, draft, tree_tokens, tree_parent, cu_nodes, u_accept, u_sample,
                      T, max_nodes: int, dtype: str,
                      requests: Optional[Sequence[int]] = None, top_k=0,
                      top_p=1.0, top_k_max=None) -> TreeBatchResult:
    """Packed trees: request b owns nodes cu[b] .. cu[b+1] - 1 and the target / draft rows
    cu[b] + b + v for its positions v = 0 .. n_b (draft rows of leaves are not read).
    T, top_k (0 or >= V: off) and top_p (>= 1 or <= 0: off) apply to every row a request
    reads: one value for every request, or one per request (T and top_p rounded to fp32);
    top_k_max bounds the active per-request top_k values, if given."""
    cu = np.asarray(cu_nodes, dtype=np.int64)
    B = cu.shape[0] - 1
    N = int(np.asarray(tree_tokens).shape[0])
    V = int(target.shape[1])
    per = lambda x, f: [f(v) for v in np.broadcast_to(np.asarray(x), (B,))]
    Ts = per(T, lambda v: float(np.float32(v)))
    ks = per(top_k, int)
    ps = per(top_p, lambda v: float(np.float32(v)))
    num_acc = np.full(B, -1, dtype=np.int32)
    num_emit = np.zeros(B, dtype=np.int32)
    out = np.full(N + B, -1, dtype=np.int32)
    nodes = np.full(N, -1, dtype=np.int32)
    errs = np.zeros(B, dtype=np.int32)
    results: List[Optional[TreeRequestResult]] = [None] * B
    bad_cu = cu[0] != 0 or cu[B] != N
    for b in (range(B) if requests is None else requests):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if bad_cu or n < 0 or n > max_nodes:
            errs[b] = ERR_K
            continue
        t_rows = _decode_rows(target[lo + b: hi + b + 1], dtype)
        d_rows = _decode_rows(draft[lo + b: hi + b + 1], dtype)
        r = tree_verify_request(t_rows, d_rows, [int(x) for x in tree_parent[lo:hi]],
                                [int(x) for x in tree_tokens[lo:hi]],
                                [float(u) for u in u_accept[lo:hi]], float(u_sample[b]), Ts[b],
                                V, ks[b], ps[b], top_k_max)
        results[b] = r
        errs[b] = r.err
        if r.a >= 0:
            num_acc[b] = r.a
            num_emit[b] = len(r.emitted)
            out[lo + b: lo + b + len(r.emitted)] = r.emitted
            nodes[lo: lo + r.a] = r.path
    return TreeBatchResult(num_acc, num_emit, out, nodes, errs, results)


def tree_commit(cache: PagedKV, num_accepted: Sequence[int], accepted_nodes: Sequence[int],
                cu_nodes: Sequence[int]) -> int:
    """Keep the accepted path in the cache layout ("Keep cache validity aligned with the
    committed token history", paragraph 3). The cycle appended n_b + 1 entries per request:
    the pending token, then node j at the pending slot + 1 + j. Path node i (i = 1..a)
    moves to the pending slot + i, in increasing i (every destination lies below every
    source still to be read); then the cache is truncated to the pending slot + 1 + a and
    blocks past the end are released, as the linear rollback does with n_b - a dropped.
    A request with a < 0, a > n_b, a path that is not strictly increasing within [0, n_b),
    or fewer than n_b + 1 entries is left as it is and flagged. Returns error bits."""
    if cache.state & KV_APPEND_REJECTED:
        return 0
    cu = [int(c) for c in cu_nodes]
    bs = cache.bs
    err = 0
    ok = [False] * cache.B
    for b in range(cache.B):
        n, a = cu[b + 1] - cu[b], int(num_accepted[b])
        path = [int(x) for x in accepted_nodes[cu[b]: cu[b] + max(a, 0)]]
        s = cache.seq_lens[b]
        good = (0 <= a <= n and s >= n + 1 and all(0 <= x < n for x in path)
                and all(path[i] < path[i + 1] for i in range(len(path) - 1)))
        if not good:
            err |= KV_ERR_ROLLBACK
            continue
        ok[b] = True
        base = s - (n + 1)                      # the pending token's slot
        for i, j in enumerate(path, start=1):
            src, dst = base + 1 + j, base + i
            if src == dst:
                continue
            Xs = int(cache.tables[b, src // bs])
            Xd = int(cache.tables[b, dst // bs])
            ds, ms = cache._block(Xs)
            dd, md = cache._block(Xd)
            dd[:, :, dst % bs] = ds[:, :, src % bs]
            md[dst % bs] = ms[src % bs]
    # truncation: the linear rollback with n_b - a entries dropped (requests left as they
    # are carry a = -1, which the rollback skips and flags)
    num = [int(num_accepted[b]) if ok[b] else -1 for b in range(cache.B)]
    err |= cache.rollback(num, cu)
    cache.err |= err
    return err
