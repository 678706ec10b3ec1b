"""GPU parity of kv_paged_append / kv_rollback against the sequential oracle: metadata
(tables, lengths, refcounts, free list, state word) and K/V bits, exactly."""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import (KVOnDevice, compare_kv_data, compare_kv_meta, dev, log, oracle_kv)
from rejection_sampling_verify_specdec_amd import binding, synth
from rejection_sampling_verify_specdec_amd.synth import KVInputs

pytestmark = pytest.mark.gpu

L, H, D = 2, 2, 8


def _bits(rng, shape):
    return rng.integers(0, 65535, size=shape, dtype=np.uint16)


def _state(B, NB, bs, MBR, seq_lens=None, rng=None, shared=None):
    """Empty-ish cache: each request gets fresh blocks for its prefix (random ids), with
    defined contents for every prefix slot. `shared`: list of (requests, n_blocks) that
    share their first n_blocks."""
    rng = rng or np.random.default_rng(0)
    perm = rng.permutation(NB).astype(np.int32)
    tables = np.full((B, MBR), -1, np.int32)
    refc = np.zeros(NB, np.int32)
    seq = np.zeros(B, np.int32) if seq_lens is None else np.array(seq_lens, np.int32)
    nxt = 0
    owner = {}
    for reqs, nblk in (shared or []):
        ids = perm[nxt:nxt + nblk]
        nxt += nblk
        for b in reqs:
            tables[b, :nblk] = ids
            refc[ids] += 1
            owner[b] = nblk
    for b in range(B):
        for lb in range(owner.get(b, 0), -(-int(seq[b]) // bs)):
            tables[b, lb] = perm[nxt]
            refc[perm[nxt]] += 1
            nxt += 1
    free = np.zeros(NB, np.int32)
    fc = NB - nxt
    free[:fc] = perm[nxt:]
    blocks = {}
    for X in np.nonzero(refc)[0]:
        blocks[int(X)] = (_bits(rng, (L, 2, bs, H, D)), np.ones(bs, bool))
    return KVInputs(L, H, D, bs, NB, MBR, tables, seq, refc, free, fc,
                    np.zeros((L, 0, H, D), np.uint16), np.zeros((L, 0, H, D), np.uint16),
                    np.zeros(B + 1, np.int32), blocks)


def _t(x, d):
    return torch.from_numpy(np.ascontiguousarray(x)).to(d)


def _kvt(x, d):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(d)


def _append(g, o, rng, n):
    d = dev()
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    kn, vn = _bits(rng, (L, int(cu[-1]), H, D)), _bits(rng, (L, int(cu[-1]), H, D))
    g.append(_kvt(kn, d), _kvt(vn, d), _t(cu, d))
    return o.append(kn, vn, cu)


def _rollback(g, o, k, a):
    d = dev()
    cu = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
    g.rollback(_t(np.asarray(a, np.int32), d), _t(cu, d))
    return o.rollback(a, cu)


def _assert_same(g, o, what, data=True):
    errs = compare_kv_meta(o, g.meta(), what)
    if data:
        errs += compare_kv_data(o, g.pool, g.kv)
    assert not errs, "\n".join(errs)


@pytest.mark.parametrize("bs", [16, 4])
def test_random_cycles(bs):
    rng = np.random.default_rng(bs)
    B, NB, MBR = 9, 1500, 200
    kv = _state(B, NB, bs, MBR, seq_lens=rng.integers(0, 40, size=B), rng=rng)
    g, o = KVOnDevice(kv, B), oracle_kv(kv)
    log(f"[kv] random cycles bs={bs}")
    for cyc in range(25):
        k = rng.integers(0, 9, size=B)
        _append(g, o, rng, k + 1)
        _assert_same(g, o, f"cycle {cyc} append", data=(cyc % 5 == 0))
        a = np.array([rng.integers(0, kk + 1) for kk in k])
        _rollback(g, o, k, a)
        _assert_same(g, o, f"cycle {cyc} rollback", data=(cyc % 5 == 4))
        o.check_invariants()


def test_copy_on_write_sharers_and_conflict():
    rng = np.random.default_rng(3)
    bs, B = 16, 6
    # requests 0..2 share two blocks, the second one partial (lengths 20, 25, 31 inside it)
    kv = _state(B, 300, bs, 40, seq_lens=[32, 32, 32, 50, 7, 0], rng=rng,
                shared=[([0, 1, 2], 2)])
    o = oracle_kv(kv)
    g = KVOnDevice(kv, B)
    # shrink the sharers' lengths inside the shared partial block (deep rollback)
    _rollback(g, o, [7, 12, 15, 0, 0, 0], [0, 0, 0, 0, 0, 0])
    _assert_same(g, o, "deep rollback")
    assert o.seq_lens[:3] == [25, 20, 17]
    # all three append: 0 and 1 copy (refcount 3, then 2), 2 writes in place over slots
    # that request 0's copy reads
    _append(g, o, rng, np.array([3, 9, 4, 2, 12, 1]))
    _assert_same(g, o, "append with copy-on-write")
    o.check_invariants()
    _rollback(g, o, [2, 8, 3, 1, 11, 0], [0, 3, 1, 1, 4, 0])
    _assert_same(g, o, "rollback after copy-on-write")
    o.check_invariants()


def test_shared_prefix_deep_rollback_keeps_blocks():
    rng = np.random.default_rng(4)
    bs, B = 16, 8
    kv = _state(B, 400, bs, 30, seq_lens=[100] * B, rng=rng,
                shared=[([0, 1, 2, 3], 4), ([4, 5, 6, 7], 4)])
    o = oracle_kv(kv)
    g = KVOnDevice(kv, B)
    shared0 = list(kv.block_tables[0, :4])
    _rollback(g, o, [0, 60, 0, 0, 0, 0, 90, 0], [0] * B)      # into / through shared blocks
    _assert_same(g, o, "deep rollback")
    assert all(o.refcount[X] >= 3 for X in shared0)
    o.check_invariants()
    _rollback(g, o, [0] * B, [0] * B)
    _assert_same(g, o, "no-op rollback")


def test_enomem_all_or_nothing_then_recover():
    rng = np.random.default_rng(5)
    bs, B = 16, 4
    kv = _state(B, 12, bs, 10, seq_lens=[16, 16, 16, 0], rng=rng)
    o = oracle_kv(kv)
    g = KVOnDevice(kv, B)
    err = _append(g, o, rng, np.array([40, 40, 40, 40]))
    assert err == oracle.KV_ERR_NOMEM
    _assert_same(g, o, "nomem")
    _rollback(g, o, [3, 3, 3, 3], [0, 0, 0, 0])               # no-op after a rejected append
    _assert_same(g, o, "rollback after nomem")
    _append(g, o, rng, np.array([2, 0, 1, 16]))
    _assert_same(g, o, "recovered append")


def test_append_invalid_capacity():
    rng = np.random.default_rng(6)
    kv = _state(3, 64, 16, 4, seq_lens=[10, 60, 0], rng=rng)
    o = oracle_kv(kv)
    g = KVOnDevice(kv, 3)
    assert _append(g, o, rng, np.array([1, 5, 1])) == oracle.KV_ERR_APPEND   # 65 > 4*16
    _assert_same(g, o, "capacity")


def test_rollback_invalid_requests_skipped():
    rng = np.random.default_rng(7)
    kv = _state(4, 64, 16, 8, seq_lens=[30, 5, 17, 40], rng=rng)
    o = oracle_kv(kv)
    g = KVOnDevice(kv, 4)
    _rollback(g, o, [3, 9, 1, 6], [-1, 2, 2, 5])   # a<0, drop>len, a>k, valid
    _assert_same(g, o, "invalid rollback")


@pytest.mark.parametrize("wl", ["c2", "c4"])
def test_full_geometry_cycle_metadata_and_bits(wl):
    # real geometry (32 layers x 8 heads x 128, block 16) and batch, decisions from the oracle
    vin = synth.make_verify(wl, seed=3, V=64)     # logits unused here: small vocabulary
    rng = np.random.default_rng(8)
    a = np.array([rng.integers(0, k + 1) for k in vin.k_b])
    kv = synth.make_kv(wl, vin, seed=3, a_hint=a)
    log(f"[kv] {wl} full geometry B={vin.B} NB={kv.num_blocks}")
    g = KVOnDevice(kv, vin.B)
    o = oracle_kv(kv)
    g.append()
    o.append(kv.k_new, kv.v_new, kv.cu_new)
    _assert_same(g, o, f"{wl} append")
    _rollback(g, o, vin.k_b, a)
    _assert_same(g, o, f"{wl} rollback")
    o.check_invariants()
