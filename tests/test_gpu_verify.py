"""GPU parity of specdec_verify against the oracle (same seeded inputs and uniforms).

Small batches are compared request by request in full; the workload sizes run the whole
batch on the GPU in the benchmark's launch configuration and compare a seeded sample of
requests with the oracle.
"""

import math

import numpy as np
import pytest
import torch

from gpu_harness import (VerifyOnDevice, compare_verify, log, oracle_verify, run_verify)
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu


def _check(vin, requests=None, **kw):
    log(f"[verify] {vin.wl.name} B={vin.B} K={vin.K} V={vin.V} {vin.dtype} T={vin.T} "
        f"top_k={vin.top_k} requests={'all' if requests is None else len(requests)}")
    g = run_verify(vin, **kw)
    o = oracle_verify(vin, requests=requests)
    rep = compare_verify(vin, g, o, requests=requests)
    log(f"[verify]   {rep}")
    rep.check()
    return g, o, rep


def test_tiny_config():
    _check(synth.make_verify("tiny", seed=0))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_many_seeds(seed):
    _check(synth.make_verify("tiny", seed=seed, B=16))


def test_c1_full_batch():
    _check(synth.make_verify("c1", seed=1))


@pytest.mark.parametrize("wl", ["c2", "c3"])
def test_full_vocab_small_batch(wl):
    # full V: several 16K-element chunks plus a ragged last chunk
    _check(synth.make_verify(wl, seed=5, B=12))


@pytest.mark.parametrize("wl,nsample", [("c2", 40), ("c3", 40)])
def test_full_size_sampled(wl, nsample):
    vin = synth.make_verify(wl, seed=0)
    reqs = sorted(np.random.default_rng(99).choice(vin.B, size=nsample, replace=False).tolist())
    _check(vin, requests=reqs)


def test_unaligned_vocab_scalar_path():
    # V * 2 bytes not a multiple of 16: the scalar-load layout
    _check(synth.make_verify("c2", seed=7, B=6, V=1001))
    _check(synth.make_verify("c1", seed=7, B=6, V=999))


def test_tiny_vocab_and_single_request():
    _check(synth.make_verify("tiny", seed=8, V=2))
    _check(synth.make_verify("tiny", seed=9, V=1, B=3))


@pytest.mark.parametrize("T", [0.05, 0.3, 2.0])
def test_temperatures(T):
    _check(synth.make_verify("c2", seed=11, B=6, V=4096, T=T))


def test_ragged_with_zero_k_requests():
    vin = synth.make_verify("c3", seed=12, B=20, V=3000, k_range=(0, 6))
    assert (vin.k_b == 0).any()
    _check(vin)


def test_max_k_64():
    _check(synth.make_verify("tiny", seed=13, B=3, V=512, k=64))


def _forced(kind):
    """c2-like batch with planted logits: rejection at a chosen position, or all accepted."""
    vin = synth.make_verify("c2", seed=21, B=4, V=2048)
    k = 5
    t32 = synth.bf16_bits_to_f32(vin.target).copy()
    d32 = synth.bf16_bits_to_f32(vin.draft).copy()
    for b, j in enumerate([0, 2, 4, k]):    # reject first, middle, last; all accepted
        lo = vin.cu_draft[b]
        for i in range(k):
            y = int(vin.draft_tokens[lo + i])
            if i < j:
                vin.u_accept[lo + i] = 0.0          # P > 0 = 0 * Q: accepted
            elif i == j:
                t32[lo + b + i, y] = -np.inf        # p(y) = 0 < q(y): rejected
    vin.target = synth.f32_to_bf16_bits(t32)
    vin.draft = synth.f32_to_bf16_bits(d32)
    return vin


def test_forced_rejection_positions_and_bonus():
    vin = _forced("positions")
    g, o, _ = _check(vin)
    assert list(g.num_accepted) == [0, 2, 4, 5]
    assert list(g.num_emitted) == [1, 3, 5, 6]


@pytest.mark.parametrize("dtype,V", [("bf16", 20000), ("f32", 4000)])
def test_repeated_proposal_ids(dtype, V):
    # "Keep cache validity aligned with the committed token history", paragraph 6: repeated
    # token ids. Every proposal of a request is one id: the argmax of its first draft row
    # (accepted often, then judged again at later positions against their own rows), or
    # token 0 for every request of the batch
    vin = synth.make_verify("c2", seed=24, B=10, V=V, dtype=dtype)
    dft = (synth.bf16_bits_to_f32(vin.draft) if dtype == "bf16" else vin.draft).reshape(vin.K, V)
    for b in range(vin.B):
        lo, hi = int(vin.cu_draft[b]), int(vin.cu_draft[b + 1])
        vin.draft_tokens[lo:hi] = int(np.argmax(dft[lo])) if b % 2 == 0 else 0
    g, o, _ = _check(vin)
    assert (g.num_accepted[::2] >= 1).any()


def test_draft_zero_probability_proposal_is_accepted_and_flagged():
    vin = synth.make_verify("c2", seed=22, B=2, V=1024)
    d32 = synth.bf16_bits_to_f32(vin.draft).copy()
    y = int(vin.draft_tokens[0])
    d32[0, y] = -np.inf                       # q(y) = 0, p(y) > 0
    vin.draft = synth.f32_to_bf16_bits(d32)
    g, o, _ = _check(vin)
    assert g.req_flags[0] & binding.ERR_QZERO and g.num_accepted[0] >= 1


def test_request_errors():
    vin = synth.make_verify("c2", seed=23, B=6, V=512)
    t32 = synth.bf16_bits_to_f32(vin.target).copy()
    d32 = synth.bf16_bits_to_f32(vin.draft).copy()
    vin.draft_tokens[vin.cu_draft[0] + 1] = 512                # token out of range
    t32[vin.cu_draft[1] + 1 + 3, 5] = np.nan                   # NaN in request 1
    d32[vin.cu_draft[2] + 2, 7] = np.inf                       # +inf in request 2 draft row
    t32[vin.cu_draft[3] + 3 + 5, :] = -np.inf                  # request 3: all -inf bonus row
    vin.u_accept[vin.cu_draft[4]] = 1.0                        # request 4: u outside [0, 1)
    vin.target = synth.f32_to_bf16_bits(t32)
    vin.draft = synth.f32_to_bf16_bits(d32)
    g, o, _ = _check(vin)
    assert list(g.num_accepted[:5]) == [-1] * 5 and g.num_accepted[5] >= 0
    exp = binding.ERR_TOKEN | binding.ERR_NONFINITE | binding.ERR_UNIFORM
    assert g.err_word & exp == exp


def test_bad_offsets_flag_every_request():
    vin = synth.make_verify("tiny", seed=24, B=3, V=64)
    v = VerifyOnDevice(vin)
    v.cu[3] = vin.K - 1                      # cu[B] != K
    v.run()
    g = v.result()
    assert (g.num_accepted == -1).all() and g.err_word & binding.ERR_K


def test_deterministic_across_runs():
    vin = synth.make_verify("c3", seed=25, B=32, V=20000)
    v = VerifyOnDevice(vin)
    v.run()
    a = v.result()
    v.out_tokens.fill_(-7)
    v.run()
    b = v.result()
    for f in ("num_accepted", "out_tokens", "p_y", "q_y", "row_sum", "resid_mass", "picked_prob"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_host_validation_einval():
    vin = synth.make_verify("tiny", seed=26, B=2, V=64)
    v = VerifyOnDevice(vin)
    with pytest.raises(binding.SpecdecError):
        v.T = 0.0
        v.run()
    v.T = 1.0
    with pytest.raises(binding.SpecdecError):
        v.max_k = 65
        v.run()
    v.max_k = vin.max_k
    small = torch.empty(8, dtype=torch.uint8, device=v.ws.device)
    with pytest.raises(binding.SpecdecError):
        binding.specdec_verify(v.tgt, v.dft, v.tokens, v.cu, v.u_acc, v.u_smp, max_k=v.max_k,
                               temperature=1.0, top_k=0, out_tokens=v.out_tokens,
                               num_accepted=v.num_acc, num_emitted=v.num_emit, err_word=v.err,
                               workspace=small)


@pytest.mark.parametrize("dtype,top_k", [("bf16", 0), ("bf16", 64), ("f32", 0), ("f32", 50)])
def test_largest_vocabulary(dtype, top_k):
    # V = 2,097,152: 256 sampling chunks; 128 (bf16) or 256 (fp32) statistics chunks
    vin = synth.make_verify("c2", seed=27, B=2, V=binding.MAX_V, k=2, dtype=dtype,
                            top_k=top_k)
    _check(vin)


@pytest.mark.parametrize("top_k", ["V-1", "V"])
def test_top_k_at_the_vocabulary_size(top_k):
    V = 3000
    vin = synth.make_verify("c4", seed=28, B=4, V=V, top_k=V - 1 if top_k == "V-1" else V)
    _check(vin)


def test_vocabulary_past_the_limit_is_einval():
    vin = synth.make_verify("tiny", seed=29, B=1, V=16)
    v = VerifyOnDevice(vin)
    lib = binding.load_library()
    st = lib.specdec_verify(v.tgt.data_ptr(), v.dft.data_ptr(), 1, v.tokens.data_ptr(),
                            v.cu.data_ptr(), v.u_acc.data_ptr(), v.u_smp.data_ptr(), 1, vin.K,
                            vin.max_k, binding.MAX_V + 1, 1.0, 0, 1.0, None, v.out_tokens.data_ptr(),
                            v.num_acc.data_ptr(), v.num_emit.data_ptr(), v.err.data_ptr(), None,
                            v.ws.data_ptr(), v.ws.numel(), None)
    assert st == binding.SPECDEC_EINVAL
