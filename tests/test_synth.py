"""Seeded input generator: determinism, layout and the recipes' structure (no GPU)."""

import numpy as np
import pytest
import torch

from rejection_sampling_verify_specdec_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)


def test_determinism_and_layout():
    a = synth.make_verify("c3", seed=3, B=16, V=512)
    b = synth.make_verify("c3", seed=3, B=16, V=512)
    assert np.array_equal(a.target, b.target) and np.array_equal(a.draft_tokens, b.draft_tokens)
    assert a.target.shape == (a.K + a.B, 512) and a.draft.shape == (a.K, 512)
    assert a.target.dtype == np.uint16 and a.cu_draft[0] == 0 and a.cu_draft[-1] == a.K
    assert ((a.k_b >= 1) & (a.k_b <= 8)).all()
    assert ((a.u_accept >= 0) & (a.u_accept < 1)).all() and a.u_accept.dtype == np.float32
    # copy class: draft rows are bitwise the target rows at the same positions
    for bb in range(a.B):
        if a.kinds[bb] == "copy":
            lo, hi = a.cu_draft[bb], a.cu_draft[bb + 1]
            assert np.array_equal(a.draft[lo:hi], a.target[lo + bb: hi + bb])
    assert sorted(set(a.kinds)) == ["copy", "noise"]


def test_draft_tokens_in_topk_set():
    v = synth.make_verify("c4", seed=1, B=4, V=2048)
    z = synth.bf16_bits_to_f32(v.draft)
    for r in range(v.K):
        thr = np.sort(z[r])[::-1][v.top_k - 1]
        assert z[r, v.draft_tokens[r]] >= thr


def test_kv_state_structure():
    v = synth.make_verify("c4", seed=2, B=8, V=256)
    kv = synth.make_kv("c4", v, seed=2, recipe=synth.KVRecipe(L=2, H=2, D=8, prefix_lo=1024,
                                                               prefix_hi=2048, share_group=4,
                                                               share_blocks=32))
    # shared blocks have refcount 4 and appear in all four tables of a group
    for g in range(2):
        for lb in range(32):
            X = kv.block_tables[4 * g, lb]
            assert kv.refcount[X] == 4
            assert all(kv.block_tables[4 * g + i, lb] == X for i in range(4))
    refs = np.zeros(kv.num_blocks, np.int64)
    for b in range(8):
        nb = -(-int(kv.seq_lens[b]) // 16)
        assert (kv.block_tables[b, :nb] >= 0).all() and (kv.block_tables[b, nb:] == -1).all()
        np.add.at(refs, kv.block_tables[b, :nb], 1)
    assert np.array_equal(refs, kv.refcount)
    free = kv.free_list[:kv.free_count]
    assert len(set(free.tolist())) == kv.free_count and (refs[free] == 0).all()
    assert kv.free_count + (refs > 0).sum() == kv.num_blocks
    assert kv.k_new.shape == (2, v.K + v.B, 2, 8)


def test_rejection_alignment_hint():
    v = synth.make_verify("c3", seed=4, B=32, V=128)
    a = np.array([min(1, k - 1) for k in v.k_b])
    kv = synth.make_kv("c3", v, seed=4, a_hint=a,
                       recipe=synth.KVRecipe(L=1, H=1, D=8, align_rejections=True))
    for b in range(v.B):
        if a[b] < v.k_b[b]:
            assert (kv.seq_lens[b] + 1 + a[b]) % 16 == 0
            assert 512 <= kv.seq_lens[b] <= 4096 + 15
