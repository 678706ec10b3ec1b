"""Oracle for the paged KV cache around a verification cycle: provisional append, rollback.

TEST INFRASTRUCTURE ONLY (see the package docstring). Sequential, in request order, on
Python lists and small NumPy arrays. Physical block contents are kept sparsely (only
blocks that a cycle reads or writes), so the oracle never materializes a whole pool.

What the pages fix:

* The target pass over the candidate block produces K/V at every processed position and
  appends them provisionally, before the accept test; after the test the cache must hold
  exactly the committed history ("Walk through KV-cache updates when speculative decoding
  rejects some draft tokens", both paragraphs).
* On a paged cache the pages covering rejected positions are freed; on a contiguous
  buffer the write pointer is rewound (same page). ``ContiguousKV`` is that second model.
* Pending-token convention: the processed prefix plus the accepted proposals are kept and
  the replacement / bonus token stays pending, so committed length = cache length + 1
  ("Keep cache validity aligned with the committed token history", paragraphs 1-2).
* A physical block may be retained with only part of it valid; invalid slots need not be
  cleared ("rejected speculative tokens remain in KV", paragraph 2; "Keep cache validity
  ...", paragraph 3).
* Block tables, ownership and reference counts decide which physical memory is valid;
  rollback of one request must not change another request's prefix, and physical sharing
  is handled by copy-on-write ("Keep cache validity ...", paragraphs 3-4).

Readings taken (the pages give the principle only):

* a cycle appends k_b + 1 entries per request: the pending last token and the k_b
  proposals, matching the k_b + 1 target logit rows;
* the free list is a LIFO stack. Append pops in ascending request order and, within a
  request, ascending logical block (a copy-on-write block first); rollback pushes in the
  same order;
* append is all-or-nothing over the batch: a bad argument or too few free blocks leaves
  every request unchanged and marks the cache so that the following rollback is a no-op;
* rollback only edits metadata (lengths, tables, refcounts, free list); stale slots keep
  their bytes;
* a shared partial block (refcount > 1) that receives new entries is first copied into a
  freshly popped block (slots below the valid length), and the old block is decref'ed;
* the draft's cache follows the draft's own processed-state convention ("Keep cache
  validity ...", paragraph 5: the draft has advanced along its own proposals and must be
  realigned with the corrected history): to propose k_b tokens the draft processed its
  pending token(s) and y_1 .. y_{k_b-1} (never y_{k_b}, which it only sampled), so after
  a_b acceptances it keeps the states of y_1 .. y_{min(a_b, k_b-1)} and drops
  max(0, k_b - 1 - a_b) entries; its pending tokens are then the correction (a_b < k_b)
  or y_{k_b} and the bonus (a_b = k_b).
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

KV_ERR_NOMEM = 64         # append needed more free blocks than available: nothing applied
KV_ERR_APPEND = 128       # append argument invalid (n_b < 0, capacity, bad offsets): nothing applied
KV_ERR_ROLLBACK = 256     # a rollback request was invalid (skipped) or metadata was corrupt
KV_APPEND_REJECTED = 1 << 16   # state bit: the last append was not applied (not sticky)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class PagedKV:
    """Sequential paged cache: block tables, seq_lens, refcounts, LIFO free list, blocks.

    ``blocks`` maps a physical block id to (data uint16 [L][2][bs][H][D], defined bool[bs])
    for every block whose contents matter; unknown slots are marked undefined.
    """

    def __init__(self, L: int, H: int, D: int, block_size: int, num_blocks: int,
                 block_tables: np.ndarray, seq_lens: Sequence[int], refcount: Sequence[int],
                 free_list: Sequence[int], free_count: int,
                 blocks: Optional[Dict[int, tuple]] = None):
        self.L, self.H, self.D, self.bs, self.NB = L, H, D, block_size, num_blocks
        self.tables = np.array(block_tables, dtype=np.int64, copy=True)
        self.MBR = self.tables.shape[1]
        self.seq_lens = [int(s) for s in seq_lens]
        self.refcount = [int(r) for r in refcount]
        self.free = [int(x) for x in list(free_list)[:free_count]]   # stack, top = last
        self.err = 0
        self.state = 0
        self.data: Dict[int, np.ndarray] = {}
        self.defined: Dict[int, np.ndarray] = {}
        for bid, (d, m) in (blocks or {}).items():
            self.data[int(bid)] = np.array(d, dtype=np.uint16, copy=True)
            self.defined[int(bid)] = np.array(m, dtype=bool, copy=True)

    # -- helpers -----------------------------------------------------------------------
    @property
    def B(self) -> int:
        return len(self.seq_lens)

    def _block(self, bid: int):
        if bid not in self.data:
            self.data[bid] = np.zeros((self.L, 2, self.bs, self.H, self.D), dtype=np.uint16)
            self.defined[bid] = np.zeros(self.bs, dtype=bool)
        return self.data[bid], self.defined[bid]

    def _pop(self) -> int:
        return self.free.pop()

    # -- provisional append ------------------------------------------------------------
    def append(self, k_new: np.ndarray, v_new: np.ndarray, cu_new: Sequence[int]) -> int:
        """Append n_b = cu_new[b+1] - cu_new[b] entries per request at slots
        seq_len .. seq_len + n_b - 1. k_new / v_new: uint16 (bf16 bits) [L][N][H][D].
        Returns the error bits raised by this call (also OR-ed into ``self.err``)."""
        cu = [int(c) for c in cu_new]
        B, bs = self.B, self.bs
        N = int(k_new.shape[1])
        ok = len(cu) == B + 1 and cu[0] == 0 and cu[B] == N
        if ok:
            for b in range(B):
                n, s = cu[b + 1] - cu[b], self.seq_lens[b]
                if n < 0 or s < 0 or _ceil_div(s + n, bs) > self.MBR:
                    ok = False
                    break
                if n > 0 and s % bs != 0:
                    X = int(self.tables[b, s // bs])
                    if X < 0 or X >= self.NB:
                        ok = False
                        break
        if not ok:
            self.err |= KV_ERR_APPEND
            self.state |= KV_APPEND_REJECTED
            return KV_ERR_APPEND
        # dry run: count pops with the copy-on-write decisions taken in order
        rc = list(self.refcount)
        need = 0
        for b in range(B):
            n, s = cu[b + 1] - cu[b], self.seq_lens[b]
            if n == 0:
                continue
            cow = s % bs != 0 and rc[int(self.tables[b, s // bs])] > 1
            if cow:
                rc[int(self.tables[b, s // bs])] -= 1
            need += (_ceil_div(s + n, bs) - _ceil_div(s, bs)) + (1 if cow else 0)
        if need > len(self.free):
            self.err |= KV_ERR_NOMEM
            self.state |= KV_APPEND_REJECTED
            return KV_ERR_NOMEM
        # apply
        for b in range(B):
            n, s = cu[b + 1] - cu[b], self.seq_lens[b]
            if n == 0:
                continue
            lb0, off = s // bs, s % bs
            if off != 0:
                old = int(self.tables[b, lb0])
                if self.refcount[old] > 1:
                    new = self._pop()
                    od, om = self._block(old)
                    nd, nm = self._block(new)
                    nd[:, :, :off] = od[:, :, :off]
                    nm[:off] = om[:off]
                    self.refcount[old] -= 1
                    self.refcount[new] = 1
                    self.tables[b, lb0] = new
            for lb in range(_ceil_div(s, bs), _ceil_div(s + n, bs)):
                new = self._pop()
                self.refcount[new] = 1
                self.tables[b, lb] = new
            for t in range(n):
                pos = s + t
                d, m = self._block(int(self.tables[b, pos // bs]))
                d[:, 0, pos % bs] = k_new[:, cu[b] + t]
                d[:, 1, pos % bs] = v_new[:, cu[b] + t]
                m[pos % bs] = True
            self.seq_lens[b] = s + n
        self.state &= ~KV_APPEND_REJECTED
        return 0

    # -- rollback to the committed prefix ----------------------------------------------
    def rollback(self, num_accepted: Sequence[int], cu_draft: Sequence[int],
                 draft: bool = False) -> int:
        """Drop trailing entries per request and free blocks past the new end: k_b - a_b for
        the target's cache (after a cycle that appended k_b + 1 entries the new length is
        the old committed prefix plus 1 + a_b: the pending token and the accepted
        proposals), max(0, k_b - 1 - a_b) for the draft's (the draft never processed
        y_{k_b})."""
        if self.state & KV_APPEND_REJECTED:
            return 0
        cu = [int(c) for c in cu_draft]
        bs = self.bs
        err = 0
        for b in range(self.B):
            k, a = cu[b + 1] - cu[b], int(num_accepted[b])
            if k < 0 or a < 0 or a > k:
                err |= KV_ERR_ROLLBACK
                continue
            s = self.seq_lens[b]
            new = s - (max(0, k - 1 - a) if draft else k - a)
            if new < 0:
                err |= KV_ERR_ROLLBACK
                continue
            for lb in range(_ceil_div(new, bs), _ceil_div(s, bs)):
                X = int(self.tables[b, lb])
                if X < 0 or X >= self.NB or self.refcount[X] <= 0:
                    err |= KV_ERR_ROLLBACK
                else:
                    self.refcount[X] -= 1
                    if self.refcount[X] == 0:
                        self.free.append(X)
                self.tables[b, lb] = -1
            self.seq_lens[b] = new
        self.err |= err
        return err

    # -- views and invariants ----------------------------------------------------------
    @property
    def free_count(self) -> int:
        return len(self.free)

    def logical_view(self, b: int, start: int = 0) -> np.ndarray:
        """K/V of request b at logical slots [start, seq_len): uint16 [L][2][n][H][D]."""
        s, bs = self.seq_lens[b], self.bs
        out = np.zeros((self.L, 2, max(s - start, 0), self.H, self.D), dtype=np.uint16)
        for pos in range(start, s):
            X = int(self.tables[b, pos // bs])
            if X not in self.data or not self.defined[X][pos % bs]:
                raise KeyError(f"request {b} slot {pos} (block {X}) has undefined contents")
            out[:, :, pos - start] = self.data[X][:, :, pos % bs]
        return out

    def check_invariants(self) -> None:
        """Conservation and ownership: every block is either on the free list exactly once
        (refcount 0) or referenced by tables exactly refcount times; tables hold -1 past
        ceil(seq_len / bs) and valid ids below it."""
        refs = [0] * self.NB
        for b in range(self.B):
            nb = _ceil_div(self.seq_lens[b], self.bs)
            for lb in range(self.MBR):
                X = int(self.tables[b, lb])
                if lb < nb:
                    assert 0 <= X < self.NB, (b, lb, X)
                    refs[X] += 1
                else:
                    assert X == -1, (b, lb, X)
        on_free = [0] * self.NB
        for X in self.free:
            on_free[X] += 1
        for X in range(self.NB):
            assert on_free[X] <= 1, ("block on free list twice", X)
            if on_free[X]:
                assert refs[X] == 0 and self.refcount[X] == 0, ("free block referenced", X)
            else:
                assert refs[X] == self.refcount[X] and refs[X] > 0, \
                    ("leak or refcount mismatch", X, refs[X], self.refcount[X])
        assert self.free_count + sum(1 for r in refs if r > 0) == self.NB


class ContiguousKV:
    """Second model: one contiguous buffer per request with a write pointer that rollback
    rewinds ("Walk through KV-cache updates ...": the contiguous alternative). With
    ``max_len`` an append that would pass it is not applied (KV_ERR_NOMEM and
    KV_APPEND_REJECTED, like the paged append), and invalid rollback requests are skipped
    and flagged."""

    def __init__(self, prefixes: List[np.ndarray], max_len: Optional[int] = None):
        # prefixes[b]: uint16 [L][2][len_b][H][D]
        self.buf = [np.array(p, dtype=np.uint16, copy=True) for p in prefixes]
        self.len = [p.shape[2] for p in prefixes]
        self.max_len = max_len
        self.state = 0

    def append(self, k_new: np.ndarray, v_new: np.ndarray, cu_new: Sequence[int]) -> int:
        B = len(self.buf)
        cu = [int(c) for c in cu_new]
        n = [cu[b + 1] - cu[b] for b in range(B)]
        self.state &= ~KV_APPEND_REJECTED
        if cu[0] != 0 or cu[B] != int(k_new.shape[1]) or any(x < 0 for x in n):
            self.state |= KV_ERR_APPEND | KV_APPEND_REJECTED
            return KV_ERR_APPEND
        if self.max_len is not None and any(self.len[b] + n[b] > self.max_len for b in range(B)):
            self.state |= KV_ERR_NOMEM | KV_APPEND_REJECTED
            return KV_ERR_NOMEM
        for b in range(B):
            lo, hi = cu[b], cu[b + 1]
            ent = np.stack([k_new[:, lo:hi], v_new[:, lo:hi]], axis=1)   # [L][2][n][H][D]
            self.buf[b] = np.concatenate([self.buf[b][:, :, :self.len[b]], ent], axis=2)
            self.len[b] += hi - lo
        return 0

    def rollback(self, num_accepted: Sequence[int], cu_draft: Sequence[int],
                 draft: bool = False) -> int:
        if self.state & KV_APPEND_REJECTED:
            return 0
        err = 0
        for b in range(len(self.buf)):
            k, a = int(cu_draft[b + 1]) - int(cu_draft[b]), int(num_accepted[b])
            drop = max(0, k - 1 - a) if draft else k - a
            if k < 0 or a < 0 or a > k or drop > self.len[b]:
                err |= KV_ERR_ROLLBACK
                continue
            self.len[b] -= drop
        self.state |= err
        return err

    def view(self, b: int, start: int = 0) -> np.ndarray:
        return self.buf[b][:, :, start:self.len[b]]
