"""GPU parity of the top-p (nucleus) transform against the oracle.

Top-p follows temperature and top-k on both sides ("Speculative decoding: accelerate LLM
generation without changing its answers", sections 3 and 4 name top-p truncation among the
transforms applied alike to p and q). Three device paths are covered:
  - top-p inside a top-k set: the nucleus is searched among the per-row merge's candidates;
  - top-p alone: each chunk gathers its largest tokens plus its max and exp-sum; the nucleus
    is searched in the complete upper set of the candidates, or, when it reaches below
    them (flat rows), by full passes over the row;
  - the generic select (top_k > 1024, tiny vocabularies, overflowing candidate lists)
    followed by the full-row nucleus passes.
Rows whose nucleus mass decision lies within NUCLEUS_MARGIN of top_p are flagged (fp32
exponentials against the oracle's fp64) and only checked for validity.
"""

import numpy as np
import pytest
import torch

from gpu_harness import VerifyOnDevice, compare_verify, log, oracle_verify
from oracle.verify import _decode_rows, transform
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu


def _redraw(vin, top_p, seed, requests=None):
    """Proposals drawn from the draft rows' transformed distributions (inside the nucleus)."""
    rng = np.random.default_rng(seed)
    reqs = range(vin.B) if requests is None else requests
    for b in reqs:
        for r in range(int(vin.cu_draft[b]), int(vin.cu_draft[b + 1])):
            z = _decode_rows(vin.draft[r:r + 1], vin.dtype)[0]
            t = transform(z, vin.T, vin.top_k, top_p)
            if t.valid:
                vin.draft_tokens[r] = int(rng.choice(vin.V, p=t.p / t.p.sum()))
    return vin


def _check(vin, top_p, requests=None, min_checked=None):
    """min_checked: requests that must be held to the full rule (default: half of them;
    the flagged count depends on the oracle's margins only, so it is fixed per case)."""
    log(f"[topp] B={vin.B} K={vin.K} V={vin.V} {vin.dtype} T={vin.T} top_k={vin.top_k} "
        f"top_p={top_p} requests={'all' if requests is None else len(requests)}")
    v = VerifyOnDevice(vin, top_p=top_p)
    v.run()
    g = v.result()
    o = oracle_verify(vin, requests=requests, top_p=top_p)
    rep = compare_verify(vin, g, o, requests=requests, top_p=top_p)
    log(f"[topp]   {rep}")
    rep.check()
    n = vin.B if requests is None else len(requests)
    assert n - rep.flagged_nucleus >= (min_checked if min_checked is not None else (n + 1) // 2)
    return g, o


@pytest.mark.parametrize("top_p", [0.3, 0.9, 0.95, 0.99, 0.999])
def test_topp_alone_bf16(top_p):
    # 0.3 and 0.9 keep tens to hundreds of tokens (the candidates hold the nucleus); 0.95
    # up to ~1700 and 0.99 thousands (one counting pass over the keys below the candidates);
    # 0.999 tens of thousands on some rows
    vin = synth.make_verify("c2", seed=60, B=6)
    _check(_redraw(vin, top_p, 61), top_p)


def test_topp_flat_rows_reach_far_below_the_candidates():
    # nearly uniform rows at top_p 0.999: the boundary lies more than 1024 keys below the
    # candidates' upper set, so the counting pass gives way to the full-row passes
    vin = synth.make_verify("c2", seed=62, B=6, target_std=0.5, classes=((1.0, "noise", 0.1),))
    _check(_redraw(vin, 0.999, 63), 0.999)


@pytest.mark.parametrize("top_p,std,V", [(0.8, 8.0, 32000), (0.9, 1.0, 4000)])
def test_topp_alone_fp32(top_p, std, V):
    # flat rows (std 1) keep most of the vocabulary: full passes; a token's probability is
    # then small, so some nucleus decisions fall within the flag margin
    vin = synth.make_verify("c1", seed=62, B=8, V=V, k=2, target_std=std)
    _check(_redraw(vin, top_p, 63), top_p, min_checked=4)


@pytest.mark.parametrize("wl,top_k", [("c4", 64), ("c1", 50), ("c4", 1000), ("c4", 2000)])
def test_topp_inside_topk(wl, top_k):
    # 2000 takes the generic select, then the full-row nucleus
    vin = synth.make_verify(wl, seed=64, B=5, top_k=top_k)
    _check(_redraw(vin, 0.9, 65), 0.9)


@pytest.mark.parametrize("V", [100, 256, 300, 4001])
def test_topp_small_and_unaligned_vocab(V):
    # V = 100: generic select; 256 and 300: one chunk whose candidate lists overflow (its
    # padding is -inf), then the generic select; 4001: unaligned rows
    vin = synth.make_verify("c4", seed=66, B=4, V=V, top_k=0)
    _check(_redraw(vin, 0.8, 67), 0.8)


def _peaked(rng, V):
    return (rng.standard_normal(V) * 6).astype(np.float32)


def _integer_ties(rng, V):
    return np.round(rng.normal(0, 2, V)).astype(np.float32)


def _signed_zeros(rng, V):
    z = -np.abs(rng.standard_normal(V).astype(np.float32)) * 4 - 0.5
    idx = rng.permutation(V)
    z[idx[:3]] = rng.normal(1.0, 0.2, 3)
    z[idx[3:400]] = np.where(rng.random(397) < 0.5, np.float32(0.0), np.float32(-0.0))
    return z


def _few_finite(rng, V):
    z = np.full(V, -np.inf, dtype=np.float32)
    z[rng.choice(V, 30, replace=False)] = rng.normal(0, 3, 30)
    return z


def _constant(rng, V):
    return np.full(V, 1.5, dtype=np.float32)


def _max_plateau(rng, V):
    z = rng.normal(0, 1, V).astype(np.float32)
    z[rng.choice(V, 5000, replace=False)] = 4.0
    return z


def _plant(vin, patterns, seed):
    rng = np.random.default_rng(seed)
    t32 = synth.bf16_bits_to_f32(vin.target).copy()
    d32 = synth.bf16_bits_to_f32(vin.draft).copy()
    for b, pat in enumerate(patterns):
        lo, hi = int(vin.cu_draft[b]), int(vin.cu_draft[b + 1])
        for r in range(lo + b, hi + b + 1):
            t32[r] = pat(rng, vin.V)
        for r in range(lo, hi):
            d32[r] = pat(rng, vin.V)
    vin.target = synth.f32_to_bf16_bits(t32)
    vin.draft = synth.f32_to_bf16_bits(d32)
    return vin


@pytest.mark.parametrize("top_k", [0, 64])
def test_topp_planted_rows(top_k):
    vin = synth.make_verify("c4", seed=68, B=6, V=32768, k=2, top_k=top_k)
    pats = [_peaked, _integer_ties, _signed_zeros, _few_finite, _constant, _max_plateau]
    _check(_redraw(_plant(vin, pats, seed=69), 0.7, 70), 0.7)


@pytest.mark.parametrize("top_p", [0.9, 0.95, 0.99])
def test_topp_full_size_sampled(top_p):
    vin = synth.make_verify("c2", seed=71)
    reqs = sorted(np.random.default_rng(72).choice(vin.B, size=16, replace=False).tolist())
    _check(_redraw(vin, top_p, 73, reqs), top_p, requests=reqs)


@pytest.mark.parametrize("off", [0.0, -0.5, 1.0, 3.0])
def test_topp_off_values_change_nothing(off):
    vin = synth.make_verify("c4", seed=74, B=8, V=20000)
    base = VerifyOnDevice(vin)
    base.run()
    g0 = base.result()
    v = VerifyOnDevice(vin, top_p=off)
    v.run()
    g1 = v.result()
    for f in ("num_accepted", "num_emitted", "out_tokens", "row_thr", "row_sum", "p_y"):
        assert np.array_equal(getattr(g0, f), getattr(g1, f)), f


def test_topp_nan_is_einval():
    vin = synth.make_verify("tiny", seed=75)
    v = VerifyOnDevice(vin)
    with pytest.raises(binding.SpecdecError):
        binding.specdec_verify(v.tgt, v.dft, v.tokens, v.cu, v.u_acc, v.u_smp, max_k=v.max_k,
                               temperature=v.T, top_k=0, out_tokens=v.out_tokens,
                               num_accepted=v.num_acc, num_emitted=v.num_emit, err_word=v.err,
                               workspace=v.ws, top_p=float("nan"))


def test_topp_deterministic():
    vin = _redraw(synth.make_verify("c2", seed=76, B=8), 0.95, 77)
    outs = []
    for _ in range(3):
        v = VerifyOnDevice(vin, top_p=0.95)
        v.run()
        g = v.result()
        outs.append((g.out_tokens.copy(), g.row_sum.copy(), g.row_thr.copy(), g.row_nkept.copy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
