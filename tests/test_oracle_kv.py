"""Pins for the paged KV oracle: a second (contiguous) model, conservation and ownership
invariants, the worked rollback example, shared-prefix isolation and copy-on-write, and
all-or-nothing failure.

Sources: "Walk through KV-cache updates when speculative decoding rejects some draft
tokens" (paragraph 1: free the pages on a paged cache, rewind the pointer on a contiguous
one); "Keep cache validity aligned with the committed token history" (paragraphs 1-4);
"rejected speculative tokens remain in KV" (paragraphs 2-3: forced rejection at a block
boundary, after preemption, under prefix reuse).
"""

import numpy as np
import pytest

from oracle.kv import (PagedKV, ContiguousKV, KV_ERR_NOMEM, KV_ERR_APPEND, KV_ERR_ROLLBACK,
                       KV_APPEND_REJECTED)

L, H, D = 2, 2, 4


def _empty(B, NB, bs, MBR, order=None):
    free = list(range(NB)) if order is None else list(order)
    return PagedKV(L, H, D, bs, NB, np.full((B, MBR), -1), [0] * B, [0] * NB, free, NB)


def _kv(rng, N):
    k = rng.integers(0, 65535, size=(L, N, H, D), dtype=np.uint16)
    v = rng.integers(0, 65535, size=(L, N, H, D), dtype=np.uint16)
    return k, v


@pytest.mark.parametrize("bs", [4, 16])
def test_paged_matches_contiguous_over_random_cycles(bs):
    rng = np.random.default_rng(bs)
    B, NB, MBR = 5, 3000, 300
    paged = _empty(B, NB, bs, MBR, order=rng.permutation(NB))
    contig = ContiguousKV([np.zeros((L, 2, 0, H, D), np.uint16) for _ in range(B)])
    for cycle in range(150):
        k = rng.integers(0, 7, size=B)
        cu = np.concatenate([[0], np.cumsum(k)])
        cu_new = cu + np.arange(B + 1)
        kn, vn = _kv(rng, int(cu_new[-1]))
        assert paged.append(kn, vn, cu_new) == 0
        contig.append(kn, vn, cu_new)
        a = np.array([rng.integers(0, kk + 1) for kk in k])
        assert paged.rollback(a, cu) == 0
        contig.rollback(a, cu)
        paged.check_invariants()
        for b in range(B):
            assert paged.seq_lens[b] == contig.len[b]
            assert np.array_equal(paged.logical_view(b), contig.view(b))
    assert paged.err == 0


def test_lifo_free_list_order_hand_example():
    # free stack bottom..top = 0..7; pops take the top, pushes go on top, both in
    # ascending request order then ascending logical block
    kv = _empty(2, 8, 4, 4)
    rng = np.random.default_rng(0)
    kn, vn = _kv(rng, 8)
    assert kv.append(kn, vn, [0, 5, 8]) == 0
    assert kv.tables[0, :2].tolist() == [7, 6] and kv.tables[1, :1].tolist() == [5]
    assert kv.free == [0, 1, 2, 3, 4]
    assert kv.rollback([0, 2], [0, 4, 6]) == 0      # request 0 drops 4 -> length 1
    assert kv.seq_lens == [1, 3] and kv.tables[0].tolist() == [7, -1, -1, -1]
    assert kv.free == [0, 1, 2, 3, 4, 6]
    kn, vn = _kv(rng, 4)
    assert kv.append(kn, vn, [0, 2, 4]) == 0
    assert kv.tables[1, :2].tolist() == [5, 6] and kv.free == [0, 1, 2, 3, 4]
    kv.check_invariants()


def test_worked_example_reject_fourth_of_five():
    # five proposals plus the pending token are appended; positions 1-3 accepted, 4
    # rejected: the cache keeps the pending token and three proposals, two are removed
    rng = np.random.default_rng(1)
    kv = _empty(1, 16, 16, 8)
    kn, vn = _kv(rng, 20)
    kv.append(kn, vn, [0, 20])
    pre = kv.logical_view(0).copy()
    kn, vn = _kv(rng, 6)
    kv.append(kn, vn, [0, 6])
    kv.rollback([3], [0, 5])
    assert kv.seq_lens[0] == 20 + 4
    view = kv.logical_view(0)
    assert np.array_equal(view[:, :, :20], pre)
    assert np.array_equal(view[:, 0, 20:], kn[:, :4]) and np.array_equal(view[:, 1, 20:], vn[:, :4])


@pytest.mark.parametrize("a", [0, 2, 4])
def test_rejection_on_block_boundary_frees_block(a):
    bs, k = 16, 5
    rng = np.random.default_rng(a)
    pre = 16 * 3 - 1 - a          # committed part after rollback ends on a block boundary
    kv = _empty(1, 32, bs, 16)
    kn, vn = _kv(rng, pre)
    kv.append(kn, vn, [0, pre])
    blocks_before = kv.NB - kv.free_count
    kn, vn = _kv(rng, k + 1)
    kv.append(kn, vn, [0, k + 1])
    assert kv.NB - kv.free_count == blocks_before + 1     # the fourth block was popped
    top = kv.free_count
    kv.rollback([a], [0, k])
    assert kv.seq_lens[0] == 48 and kv.seq_lens[0] % bs == 0
    assert kv.NB - kv.free_count == blocks_before          # and freed again
    assert kv.free_count == top + 1 and kv.tables[0, 3] == -1
    kv.check_invariants()


def _shared_state(rng, bs=4, n_share=2, B=4, tail=3, NB=64, MBR=16):
    """B requests sharing n_share full blocks (refcount B), each with its own tail."""
    kv = _empty(B, NB, bs, MBR)
    shared = [kv.free.pop() for _ in range(n_share)]
    blocks = {}
    for X in shared:
        kv.refcount[X] = B
        blocks[X] = rng.integers(0, 65535, size=(L, 2, bs, H, D), dtype=np.uint16)
    for b in range(B):
        for lb, X in enumerate(shared):
            kv.tables[b, lb] = X
        kv.seq_lens[b] = n_share * bs
    for X, d in blocks.items():
        kv.data[X] = d
        kv.defined[X] = np.ones(bs, dtype=bool)
    kn, vn = _kv(rng, B * tail)
    kv.append(kn, vn, [t * tail for t in range(B + 1)])
    kv.check_invariants()
    return kv, shared


def test_shared_prefix_isolation_and_deep_rollback():
    rng = np.random.default_rng(2)
    kv, shared = _shared_state(rng)
    views = [kv.logical_view(b).copy() for b in range(4)]
    free_before = list(kv.free)
    tail1 = int(kv.tables[1, 2])
    # preemption-like deep rollback of request 1 to length 5 (inside the second shared block)
    cu = [0, 0, 6, 6, 6]
    assert kv.rollback([0, 0, 0, 0], cu) == 0
    assert kv.seq_lens[1] == 5
    assert kv.refcount[shared[0]] == 4 and kv.refcount[shared[1]] == 4
    assert kv.free == free_before + [tail1]
    # request 1's private tail block went back to the free list; shared ones did not
    assert all(X not in kv.free for X in shared)
    for b in (0, 2, 3):
        assert np.array_equal(kv.logical_view(b), views[b])
    assert np.array_equal(kv.logical_view(1), views[1][:, :, :5])
    kv.check_invariants()
    # roll request 1 back into the first shared block: second shared block decref'ed, kept
    assert kv.rollback([0, 0, 0, 0], [0, 0, 2, 2, 2]) == 0
    assert kv.seq_lens[1] == 3 and kv.refcount[shared[1]] == 3 and shared[1] not in kv.free
    kv.check_invariants()
    # appending into the shared partial block copies it first (copy-on-write)
    kn, vn = _kv(rng, 2)
    assert kv.append(kn, vn, [0, 0, 2, 2, 2]) == 0
    X = int(kv.tables[1, 0])
    assert X != shared[0] and kv.refcount[shared[0]] == 3 and kv.refcount[X] == 1
    for b in (0, 2, 3):
        assert np.array_equal(kv.logical_view(b), views[b])
    v1 = kv.logical_view(1)
    assert np.array_equal(v1[:, :, :3], views[1][:, :, :3])
    assert np.array_equal(v1[:, 0, 3:], kn) and np.array_equal(v1[:, 1, 3:], vn)
    kv.check_invariants()


def test_cow_sharers_in_one_batch():
    # requests 0 and 1 share a partial block (refcount 2): the first copies, the second
    # then holds the only reference and writes in place
    rng = np.random.default_rng(3)
    bs = 4
    kv = _empty(2, 16, bs, 8)
    X = kv.free.pop()
    kv.refcount[X] = 2
    kv.data[X] = rng.integers(0, 65535, size=(L, 2, bs, H, D), dtype=np.uint16)
    kv.defined[X] = np.array([True, True, False, False])
    for b in range(2):
        kv.tables[b, 0] = X
        kv.seq_lens[b] = 2
    kv.check_invariants()
    old = kv.data[X].copy()
    kn, vn = _kv(rng, 4)
    top = kv.free[-1]
    assert kv.append(kn, vn, [0, 2, 4]) == 0
    assert kv.tables[0, 0] == top and kv.tables[1, 0] == X
    assert kv.refcount[X] == 1 and kv.refcount[top] == 1
    assert np.array_equal(kv.logical_view(0)[:, :, :2], old[:, :, :2])
    assert np.array_equal(kv.logical_view(1)[:, :, :2], old[:, :, :2])
    assert np.array_equal(kv.logical_view(0)[:, 0, 2:], kn[:, :2])
    assert np.array_equal(kv.logical_view(1)[:, 0, 2:], kn[:, 2:])
    kv.check_invariants()


def test_enomem_is_all_or_nothing_and_blocks_rollback():
    rng = np.random.default_rng(4)
    kv = _empty(3, 4, 4, 8)
    kn, vn = _kv(rng, 12)
    assert kv.append(kn, vn, [0, 4, 8, 12]) == 0      # uses 3 of 4 blocks
    snap = (kv.tables.copy(), list(kv.seq_lens), list(kv.refcount), list(kv.free))
    kn, vn = _kv(rng, 6)
    assert kv.append(kn, vn, [0, 2, 4, 6]) == KV_ERR_NOMEM   # needs 3 more, 1 free
    assert kv.state & KV_APPEND_REJECTED and kv.err & KV_ERR_NOMEM
    assert np.array_equal(kv.tables, snap[0]) and kv.seq_lens == snap[1]
    assert kv.refcount == snap[2] and kv.free == snap[3]
    assert kv.rollback([0, 0, 0], [0, 1, 2, 3]) == 0 and kv.seq_lens == snap[1]
    kn, vn = _kv(rng, 1)
    assert kv.append(kn, vn, [0, 1, 1, 1]) == 0 and not kv.state & KV_APPEND_REJECTED
    kv.check_invariants()


def test_append_bad_arguments_change_nothing():
    rng = np.random.default_rng(5)
    kv = _empty(2, 8, 4, 2)
    kn, vn = _kv(rng, 4)
    assert kv.append(kn, vn, [0, 3, 2]) == KV_ERR_APPEND      # n_1 < 0 / cu[B] != N
    kn, vn = _kv(rng, 9)
    assert kv.append(kn, vn, [0, 9, 9]) == KV_ERR_APPEND      # 9 slots > 2 blocks of 4
    assert kv.seq_lens == [0, 0] and kv.free_count == 8


def test_rollback_invalid_requests_are_skipped():
    rng = np.random.default_rng(6)
    kv = _empty(3, 16, 4, 8)
    kn, vn = _kv(rng, 9)
    kv.append(kn, vn, [0, 3, 6, 9])
    err = kv.rollback([3, -1, 1], [0, 2, 4, 6])    # a > k for 0, a < 0 for 1
    assert err == KV_ERR_ROLLBACK
    assert kv.seq_lens == [3, 3, 2]
    err = kv.rollback([0, 0, 0], [0, 4, 4, 4])      # drop 4 > length 3
    assert err == KV_ERR_ROLLBACK and kv.seq_lens[0] == 3
    kv.check_invariants()


def test_repeated_cycles_do_not_leak_with_sharing():
    rng = np.random.default_rng(7)
    kv, shared = _shared_state(rng, B=4, tail=1, NB=2000, MBR=200)
    for _ in range(100):
        k = rng.integers(0, 6, size=4)
        cu = np.concatenate([[0], np.cumsum(k)])
        kn, vn = _kv(rng, int(cu[-1]) + 4)
        assert kv.append(kn, vn, cu + np.arange(5)) == 0
        a = np.array([rng.integers(0, kk + 1) for kk in k])
        assert kv.rollback(a, cu) == 0
        kv.check_invariants()
    assert all(kv.refcount[X] == 4 for X in shared)


# ---------------------------------------------------------------------------------------
# Target and draft caches over many rounds ("Keep cache validity aligned with the committed
# token history", paragraphs 1-2 and 5-6): after every round each cache must hold exactly
# the states its model computes for the committed history (no contamination), as long a
# prefix of it as that model has processed (no lost state), and no block may leak.
# ---------------------------------------------------------------------------------------

def _state(model, b, pos, tok):
    """K/V a model computes at position pos of request b for token tok (stand-in values)."""
    r = np.random.default_rng([model, b, pos, tok])
    return r.integers(0, 0x7f00, size=(L, 2, H, D), dtype=np.uint16)


def _entries(model, b, pos0, toks):
    return np.stack([_state(model, b, pos0 + i, t) for i, t in enumerate(toks)], axis=2) \
        if toks else np.zeros((L, 2, 0, H, D), np.uint16)


def _append_all(cache, ents):
    """Append per-request entry stacks [L][2][n][H][D] in one batched call."""
    n = [e.shape[2] for e in ents]
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    k = np.concatenate([e[:, 0] for e in ents], axis=1) if cu[-1] else np.zeros((L, 0, H, D), np.uint16)
    v = np.concatenate([e[:, 1] for e in ents], axis=1) if cu[-1] else np.zeros((L, 0, H, D), np.uint16)
    assert cache.append(k, v, cu) == 0
    return cu


@pytest.mark.parametrize("seed", [0, 1])
def test_target_and_draft_caches_track_the_committed_history(seed):
    rng = np.random.default_rng(100 + seed)
    B, NB, MBR, bs, V = 6, 4000, 400, 4, 50
    tgt = _empty(B, NB, bs, MBR, order=rng.permutation(NB))
    dft = _empty(B, NB, bs, MBR, order=rng.permutation(NB))
    hist = [[int(rng.integers(V))] for _ in range(B)]     # the prompt's last token is pending
    for rnd in range(40):
        k = rng.integers(0, 6, size=B)
        y = [list(rng.integers(V, size=int(k[b]))) for b in range(B)]
        a = np.array([int(rng.integers(0, k[b] + 1)) for b in range(B)])
        # drafting: the draft processes its pending tokens, then y_1 .. y_{k-1}
        d0 = list(dft.seq_lens)
        _append_all(dft, [_entries(1, b, d0[b], hist[b][d0[b]:] + y[b][:-1]) if k[b] else
                          _entries(1, b, d0[b], []) for b in range(B)])
        # verification pass: the target processes the pending token and y_1 .. y_k
        t0 = list(tgt.seq_lens)
        _append_all(tgt, [_entries(0, b, t0[b], [hist[b][-1]] + y[b]) for b in range(B)])
        cu = np.concatenate([[0], np.cumsum(k)])
        assert tgt.rollback(a, cu) == 0
        assert dft.rollback(a, cu, draft=True) == 0
        for b in range(B):
            hist[b] += y[b][:a[b]] + [int(rng.integers(V))]     # accepted, then x*
        for b in range(B):
            n = len(hist[b])
            assert tgt.seq_lens[b] == n - 1                      # one token pending
            want = _entries(0, b, 0, hist[b][:n - 1])
            assert np.array_equal(tgt.logical_view(b), want)
            # the draft keeps every state it computed on the committed history
            if k[b]:
                keep = d0[b] + (t0[b] + 1 - d0[b]) + min(a[b], k[b] - 1)
            else:
                keep = d0[b]
            assert dft.seq_lens[b] == keep, (rnd, b)
            assert keep <= n - 1
            assert np.array_equal(dft.logical_view(b), _entries(1, b, 0, hist[b][:keep]))
        tgt.check_invariants()
        dft.check_invariants()


def test_contiguous_capacity_all_or_nothing_and_invalid_rollbacks():
    from oracle.kv import KV_APPEND_REJECTED
    pre = [np.zeros((1, 2, n, 1, 2), np.uint16) for n in (3, 9)]
    c = ContiguousKV(pre, max_len=10)
    k = np.ones((1, 3, 1, 2), np.uint16)
    # request 1 would hold 11 entries: nothing applied
    assert c.append(k, k, [0, 1, 3]) == KV_ERR_NOMEM and c.len == [3, 9]
    assert c.state & KV_APPEND_REJECTED
    assert c.rollback([0, 0], [0, 1, 2]) == 0 and c.len == [3, 9]      # no-op after it
    assert c.append(k[:, :2], k[:, :2], [0, 1, 2]) == 0 and c.len == [4, 10]
    # a > k is skipped and flagged; the valid request rewinds
    assert c.rollback([2, 0], [0, 1, 2]) == KV_ERR_ROLLBACK and c.len == [4, 9]
