"""Randomized GPU parity sweep: seeded random batches that mix every option the
verification step takes (dtype, vocabulary alignment, batch size, ragged and empty
proposal counts, temperature, top-k, top-p, per-request parameters, stopping), each
checked against the oracle under the flagged-margin rule, with the acceptance rates of the
same launch where no nucleus boundary is too close to call; and the fused cycle against the
three calls bit for bit on a further set. A failure prints the case's seed and options.
"""

import os

import numpy as np
import pytest

from gpu_harness import VerifyOnDevice, compare_verify, log, oracle_verify
from rejection_sampling_verify_specdec_amd import synth
from test_gpu_analytics import _compare as compare_analytics
from test_gpu_cycle import _run_mode

pytestmark = pytest.mark.gpu


def _seeds(n):
    """The committed seeds 0 .. n-1, or SPECDEC_RANDOM_SEEDS="start:count" for a longer sweep
    (every case reproducible from its seed)."""
    spec = os.environ.get("SPECDEC_RANDOM_SEEDS")
    if not spec:
        return list(range(n))
    start, count = (int(x) for x in spec.split(":"))
    return list(range(start, start + count))


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = "bf16" if r.random() < 0.6 else "f32"
    V = int(r.choice([97, 1000, 4096, 5003, 16384, 40000]))
    B = int(r.integers(1, 24))
    kmax = int(r.integers(0, 9))
    opts = dict(
        dtype=dtype, V=V, B=B, k_range=(0, kmax) if kmax else None, k=kmax,
        T=float(r.choice([0.3, 0.7, 1.0, 1.6])),
        top_k=int(r.choice([0, 0, 1, 8, 64, 300, V - 1, V])),
        top_p=float(r.choice([1.0, 1.0, 0.5, 0.9, 0.99])),
        per_request=bool(r.random() < 0.3),
        stop=bool(r.random() < 0.3),
        noise=float(r.choice([0.2, 1.0, 2.0])),
    )
    return opts, r


def _inputs(opts, seed):
    wl = synth.WORKLOADS["c1"]
    over = dict(dtype=opts["dtype"], T=opts["T"], top_k=opts["top_k"], k=max(opts["k"], 1),
                k_range=opts["k_range"], classes=((1.0, "noise", opts["noise"]),),
                target_std=2.5)
    return synth.make_verify(wl, seed=seed, B=opts["B"], V=opts["V"], **over)


@pytest.mark.parametrize("seed", _seeds(64))
def test_random_batches_match_the_oracle(seed):
    opts, r = _case(seed)
    vin = _inputs(opts, seed)
    log(f"[random] seed {seed}: {opts} K={vin.K}")
    kw, okw = {}, {}
    T, k, p = vin.T, vin.top_k, opts["top_p"]
    if opts["per_request"]:
        Ts = r.choice([0.4, 0.8, 1.2], vin.B).astype(np.float32)
        ks = r.choice([0, 4, 50, vin.V], vin.B).astype(np.int32)
        ps = r.choice([1.0, 0.8, 0.95], vin.B).astype(np.float32)
        kw.update(temps=Ts, top_ks=ks, top_ps=ps, top_k_max=64)
        okw.update(T=Ts, top_k=ks, top_p=ps, top_k_max=64)
        T, k, p = Ts, ks, ps
    else:
        kw.update(top_p=p)
        okw.update(top_p=p)
    if opts["stop"]:
        eos = r.integers(0, vin.V, vin.B).astype(np.int32)
        # make some EOS tokens likely: a request's own first proposal
        for b in range(vin.B):
            lo, hi = int(vin.cu_draft[b]), int(vin.cu_draft[b + 1])
            if hi > lo and r.random() < 0.5:
                eos[b] = vin.draft_tokens[lo]
        cap = r.integers(0, 5, vin.B).astype(np.int32)
        kw.update(eos=eos, max_emit=cap)
        okw.update(eos=eos, max_emit=cap)
    v = VerifyOnDevice(vin, analytics=True, **kw)
    v.run()
    g = v.result()
    o = oracle_verify(vin, **okw)
    rep = compare_verify(vin, g, o, T=T, top_k=k, top_p=p, eos=okw.get("eos"),
                         max_emit=okw.get("max_emit"))
    log(f"[random]   {rep}")
    assert not rep.errors, f"seed {seed} {opts}\n" + "\n".join(rep.errors)
    rep.check()
    if not opts["stop"] and rep.flagged_nucleus == 0:
        # acceptance rates of the same batch (a nucleus boundary too close to call moves a
        # kept token, and with it beta; a stopped request's expectation is not capped)
        compare_analytics(vin, g, T=T, top_k=k, top_p=p,
                          top_k_max=okw.get("top_k_max"))


@pytest.mark.parametrize("seed", _seeds(12))
def test_random_fused_cycles_equal_three_calls(seed):
    opts, _ = _case(100 + seed)
    opts["V"] = max(opts["V"], 1000)
    vin = _inputs(opts, 100 + seed)
    rec = synth.KVRecipe(L=2, H=2, D=8, prefix_lo=10, prefix_hi=200, share_group=2,
                         share_blocks=1)
    kv = synth.make_kv("c1", vin, seed=seed, recipe=rec)
    log(f"[random-fused] seed {seed}: {opts} K={vin.K}")
    a = _run_mode(vin, kv, "calls", top_p=opts["top_p"])
    b = _run_mode(vin, kv, "fused", top_p=opts["top_p"])
    for f in ("num_accepted", "num_emitted", "out_tokens", "err_word", "p_y", "q_y", "row_sum",
              "row_thr", "row_nkept", "resid_mass", "picked_prob", "req_flags"):
        assert np.array_equal(np.asarray(getattr(a[0], f)), np.asarray(getattr(b[0], f))), f
    for f in ("tables", "seq_lens", "refcount", "free_list", "free_count", "state"):
        assert np.array_equal(np.asarray(a[1][f]), np.asarray(b[1][f])), f
    assert np.array_equal(a[2], b[2])


@pytest.mark.parametrize("seed", _seeds(16))
def test_random_trees_match_the_oracle_for_any_team(seed):
    # random tree batches (sizes, vocabulary, dtype, temperature, top-k, top-p, branching,
    # draft noise, empty trees) with a random team size: checked against the oracle, and
    # bit for bit against a team of one
    from test_gpu_tree import TreeOnDevice, compare_tree
    import oracle
    r = np.random.default_rng(2000 + seed)
    nlo = int(r.integers(0, 6))
    kw = dict(B=int(r.integers(1, 13)), V=int(r.choice([97, 1000, 4001, 16384, 40000])),
              dtype="bf16" if r.random() < 0.6 else "f32", T=float(r.choice([0.5, 1.0, 1.5])),
              n_range=(nlo, nlo + int(r.integers(0, 30))), branch=float(r.choice([0.0, 0.5, 1.0])),
              noise_std=float(r.choice([0.1, 0.5, 2.0])), target_std=float(r.choice([1.0, 3.0])))
    team = int(r.choice([0, 2, 3, 7, 16]))
    top_k = int(r.choice([0, 0, 1, 8, 64, 300, 2000]))
    top_p = float(r.choice([1.0, 1.0, 0.5, 0.9, 0.99]))
    tin = synth.make_tree(seed=3000 + seed, top_k=top_k, **kw)
    pr = {}
    if r.random() < 0.4:              # per-request arrays (some requests the multi-pass select)
        B = tin.B
        pr = dict(temps=r.choice([0.5, 1.0, 1.5], B).astype(np.float32),
                  top_ks=r.choice([0, 8, 64, 2000, kw["V"]], B).astype(np.int32),
                  top_ps=r.choice([1.0, 0.9, 0.5], B).astype(np.float32), top_k_max=2000)
    log(f"[random-tree] seed {seed}: {kw} N={tin.N} team {team} top_k {top_k} top_p {top_p} "
        f"per-request {bool(pr)}")
    g = TreeOnDevice(tin, team=team, ws_fill=0x5A, top_k=top_k, top_p=top_p, **pr).run()
    T = pr.get("temps", tin.T)
    k = pr.get("top_ks", top_k)
    p = pr.get("top_ps", top_p)
    o = oracle.tree_verify_batch(tin.target, tin.draft, tin.tokens, tin.parent, tin.cu_nodes,
                                 tin.u_accept, tin.u_sample, T, tin.max_nodes, tin.dtype,
                                 top_k=k, top_p=p, top_k_max=pr.get("top_k_max"))
    errs, fl, mism = compare_tree(tin, g, o, k, p, T)
    log(f"[random-tree]   flagged {fl}, flagged mismatches {mism}")
    assert not errs, f"seed {seed} {kw} team {team}\n" + "\n".join(errs[:20])
    solo = TreeOnDevice(tin, team=1, top_k=top_k, top_p=top_p, **pr).run()
    for key in ("a", "n", "out", "nodes", "flags"):
        assert np.array_equal(g[key], solo[key]), key


@pytest.mark.parametrize("seed", _seeds(12))
def test_random_early_exit_cycles_equal_the_full_cycle(seed):
    # the early-exit cycle on random batches (dtype, V, B, ragged and empty k_b, top-k,
    # top-p, scalar or per-request parameters with an invalid temperature now and then,
    # EOS / caps, draft noise): against the oracle, and bit for bit against the full cycle
    # on twin caches
    from test_gpu_early_exit import _both
    opts, r = _case(200 + seed)
    vin = _inputs(opts, 200 + seed)
    rec = synth.KVRecipe(L=2, H=2, D=8, prefix_lo=10, prefix_hi=200, share_group=2,
                         share_blocks=1)
    kv = synth.make_kv("c1", vin, seed=seed, recipe=rec)
    kw = dict(top_p=opts["top_p"])
    if opts["per_request"]:
        temps = r.choice([0.4, 0.8, 1.2], vin.B).astype(np.float32)
        if r.random() < 0.5:
            temps[int(r.integers(0, vin.B))] = 0.0
        kw["temps"] = temps
        if r.random() < 0.5:
            kw.update(top_ks=r.choice([0, 4, 50, vin.V], vin.B).astype(np.int32),
                      top_ps=r.choice([1.0, 0.8, 0.95], vin.B).astype(np.float32),
                      top_k_max=64)
    if opts["stop"]:
        eos = r.integers(0, vin.V, vin.B).astype(np.int32)
        for b in range(vin.B):
            lo, hi = int(vin.cu_draft[b]), int(vin.cu_draft[b + 1])
            if hi > lo and r.random() < 0.5:
                eos[b] = vin.draft_tokens[lo]
        kw.update(eos=eos, max_emit=r.integers(0, 5, vin.B).astype(np.int32))
    log(f"[random-early] seed {seed}: {opts} K={vin.K}")
    _both(vin, kv, **kw)


@pytest.mark.parametrize("seed", [209, 879, 1015, 1990])
def test_zero_residual_draw_falls_back_like_the_oracle(seed):
    # cases found by extended sweeps: top-p keeps kept sets with the same logit differences
    # in a request's target and draft rows and the proposal lies outside them, so the
    # residual is exactly zero and both sides draw from p and flag it; 1015: a small
    # residual mass, drawn from on both sides (the device re-derives small residuals with
    # its precise arithmetic)
    test_random_batches_match_the_oracle(seed)
