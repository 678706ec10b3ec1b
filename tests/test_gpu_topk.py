"""GPU parity of the top-k transform against the oracle.

Rows take the chunked select (per-chunk candidate lists, then a per-row merge); top_k
above 1024, rows holding NaN/+inf and rows with a chunk whose candidates overflow its
capacity (heavy ties at the threshold) take the generic multi-pass select. Both must give
the oracle's threshold, kept count, max and exp-sum on every row, and the same decisions
and tokens.
"""

import numpy as np
import pytest

from gpu_harness import compare_verify, log, oracle_verify, run_verify
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu


def _check(vin, requests=None):
    log(f"[topk] B={vin.B} K={vin.K} V={vin.V} {vin.dtype} T={vin.T} top_k={vin.top_k} "
        f"requests={'all' if requests is None else len(requests)}")
    g = run_verify(vin)
    o = oracle_verify(vin, requests=requests)
    rep = compare_verify(vin, g, o, requests=requests)
    log(f"[topk]   {rep}")
    rep.check()
    return g, o


def test_topk_full_vocab_small_batch():
    _check(synth.make_verify("c4", seed=41, B=8))


def test_topk_full_size_sampled():
    vin = synth.make_verify("c4", seed=0)
    reqs = sorted(np.random.default_rng(98).choice(vin.B, size=24, replace=False).tolist())
    _check(vin, requests=reqs)


def test_topk_fp32_rows():
    _check(synth.make_verify("c1", seed=42, B=8, top_k=50))


@pytest.mark.parametrize("top_k", [1, 2, 1000, 1024, 1025])
def test_topk_values(top_k):
    # 1000 and 1024 bound the chunk threshold by per-group maxima; 1025 is generic
    _check(synth.make_verify("c4", seed=43, B=4, V=16384, top_k=top_k))


def test_topk_unaligned_vocab():
    _check(synth.make_verify("c4", seed=44, B=4, V=4001))


def _kth_largest(z, k):
    return float(np.partition(z, z.size - k)[z.size - k])


def _plant(vin, patterns, seed):
    """Replace every row of request b by a fresh draw of patterns[b] (a callable of rng and
    V) and redraw its proposals among the draft row's kept tokens."""
    rng = np.random.default_rng(seed)
    t32 = synth.bf16_bits_to_f32(vin.target).copy()
    d32 = synth.bf16_bits_to_f32(vin.draft).copy()
    for b, pat in enumerate(patterns):
        if pat is None:
            continue
        lo, hi = int(vin.cu_draft[b]), int(vin.cu_draft[b + 1])
        for r in range(lo + b, hi + b + 1):
            t32[r] = pat(rng, vin.V)
        for r in range(lo, hi):
            d32[r] = pat(rng, vin.V)
            finite = np.isfinite(d32[r])
            z = np.where(finite, d32[r], -np.inf)
            thr = _kth_largest(z, vin.top_k)
            cand = np.flatnonzero((z >= thr) & (z > -np.inf))
            vin.draft_tokens[r] = int(rng.choice(cand)) if cand.size else 0
    vin.target = synth.f32_to_bf16_bits(t32)
    vin.draft = synth.f32_to_bf16_bits(d32)
    return vin


def _signed_zero_threshold(rng, V):
    # 40 positives, 100 zeros of either sign, the rest negative: the 64th largest is 0
    z = -np.abs(rng.standard_normal(V).astype(np.float32)) * 3 - 0.01
    idx = rng.permutation(V)
    z[idx[:40]] = rng.normal(5, 1, 40)
    z[idx[40:140]] = np.where(rng.random(100) < 0.5, np.float32(0.0), np.float32(-0.0))
    return z


def _few_finite(rng, V):
    # 30 finite logits and -inf elsewhere: fewer than top_k tokens can be kept
    z = np.full(V, -np.inf, dtype=np.float32)
    z[rng.choice(V, 30, replace=False)] = rng.normal(0, 3, 30)
    return z


def _integer_ties(rng, V):
    return np.round(rng.normal(0, 3, V)).astype(np.float32)


def _ascending(rng, V):
    # the largest logits sit in consecutive tokens, a few threads' registers
    return np.sort(rng.normal(0, 3, V)).astype(np.float32)


def _constant(rng, V):
    return np.full(V, 1.5, dtype=np.float32)


def _max_plateau(rng, V):
    # 5000 tokens share the maximum: more candidates than the list holds
    z = rng.normal(0, 1, V).astype(np.float32)
    z[rng.choice(V, 5000, replace=False)] = 4.0
    return z


def test_topk_planted_rows_small_vocab():
    vin = synth.make_verify("c4", seed=45, B=6, V=4096, k=3)
    pats = [_signed_zero_threshold, _few_finite, _integer_ties, _ascending, _constant, None]
    _check(_plant(vin, pats, seed=46))


def test_topk_planted_rows_one_chunk():
    # every token a candidate (threshold -inf, signed zeros) without overflowing the chunk
    vin = synth.make_verify("c4", seed=50, B=3, V=256, k=2)
    pats = [_few_finite, _signed_zero_threshold, _integer_ties]
    _check(_plant(vin, pats, seed=51))


def test_topk_planted_rows_large_vocab():
    vin = synth.make_verify("c4", seed=47, B=5, V=32768, k=2)
    pats = [_constant, _max_plateau, _ascending, _integer_ties, _signed_zero_threshold]
    _check(_plant(vin, pats, seed=48))


def test_topk_nonfinite_rows():
    vin = synth.make_verify("c4", seed=49, B=4, V=8192, k=3)
    t = vin.target.copy()
    d = vin.draft.copy()
    t[int(vin.cu_draft[0]) + 0 + 1, 100] = 0x7FC0       # +NaN in a target row
    d[int(vin.cu_draft[1]) + 2, 5] = 0xFFC1             # -NaN in a draft row
    t[int(vin.cu_draft[2]) + 2 + 0, 7] = 0x7F80         # +inf
    t[int(vin.cu_draft[3]) + 3 + 1, :50] = 0xFF80       # -inf is a valid logit
    vin.target, vin.draft = t, d
    g, _ = _check(vin)
    assert list(g.num_accepted[:3]) == [-1, -1, -1] and g.num_accepted[3] >= 0
    assert g.err_word & binding.ERR_NONFINITE
