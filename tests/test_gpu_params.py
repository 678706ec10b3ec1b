"""GPU parity with per-request temperature / top-k / top-p ("Speculative decoding:
accelerate LLM generation without changing its answers", sections 3 and 4: one transform
for p and q of a request; requests of a batch may differ).

Each request's rows take its own parameters: unfiltered rows the plain statistics, top-k
rows the candidate select (or the multi-pass select above 1024), top-p rows the nucleus.
A request with invalid parameters fails alone with SPECDEC_ERR_PARAM.
"""

import numpy as np
import pytest
import torch

from gpu_harness import (KVOnDevice, VerifyOnDevice, compare_kv_meta, compare_verify, log,
                         oracle_kv, oracle_verify)
from oracle.verify import _decode_rows, transform
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu


def _redraw(vin, Ts, ks, ps, seed, requests=None):
    """Proposals drawn from each request's transformed draft rows."""
    rng = np.random.default_rng(seed)
    for b in (range(vin.B) if requests is None else requests):
        if not (Ts[b] > 0 and np.isfinite(Ts[b])) or np.isnan(ps[b]):
            continue
        for r in range(int(vin.cu_draft[b]), int(vin.cu_draft[b + 1])):
            z = _decode_rows(vin.draft[r:r + 1], vin.dtype)[0]
            t = transform(z, float(np.float32(Ts[b])), int(ks[b]), float(np.float32(ps[b])))
            if t.valid:
                vin.draft_tokens[r] = int(rng.choice(vin.V, p=t.p / t.p.sum()))
    return vin


def _check(vin, Ts, ks, ps, top_k_max=None, requests=None, redraw=True, seed=0):
    B = vin.B
    Ts = np.broadcast_to(np.asarray(Ts, np.float64), (B,))
    ks = np.broadcast_to(np.asarray(ks, np.int64), (B,))
    ps = np.broadcast_to(np.asarray(ps, np.float64), (B,))
    if redraw:
        _redraw(vin, Ts, ks, ps, seed, requests)
    log(f"[params] B={B} K={vin.K} V={vin.V} {vin.dtype} T={list(np.round(Ts, 3))} "
        f"top_k={list(ks)} top_p={list(ps)} top_k_max={top_k_max}")
    v = VerifyOnDevice(vin, temps=Ts, top_ks=ks, top_ps=ps,
                       top_k_max=top_k_max if top_k_max is not None else int(max(ks.max(), 0)))
    v.run()
    g = v.result()
    o = oracle_verify(vin, requests=requests, T=Ts, top_k=ks, top_p=ps,
                      top_k_max=top_k_max if top_k_max is not None else int(max(ks.max(), 0)))
    rep = compare_verify(vin, g, o, requests=requests, T=Ts, top_k=ks, top_p=ps)
    log(f"[params]   {rep}")
    rep.check()
    return g, o


def test_per_request_temperature_bf16():
    vin = synth.make_verify("c2", seed=80, B=8)
    _check(vin, [0.3, 0.5, 0.7, 0.7, 1.0, 1.3, 2.0, 0.05], 0, 1.0, seed=81)


def test_per_request_temperature_fp32():
    vin = synth.make_verify("c1", seed=82, B=8)
    _check(vin, np.linspace(0.2, 1.8, 8), 0, 1.0, seed=83)


def test_mixed_transforms_bf16():
    # unfiltered, top-k small / at the group limit / generic / off (>= V, <= 0), top-p alone
    # and inside top-k, in one batch
    vin = synth.make_verify("c4", seed=84, B=10)
    V = vin.V
    Ts = [0.8, 0.6, 1.0, 0.9, 0.7, 1.2, 0.8, 0.5, 1.0, 0.75]
    ks = [0, 1, 64, 1000, 2000, V, -3, 0, 50, 64]
    ps = [1.0, 1.0, 1.0, 0.9, 1.0, 1.0, 0.0, 0.9, 0.6, 0.95]
    _check(vin, Ts, ks, ps, top_k_max=2000, seed=85)


def test_mixed_transforms_fp32():
    vin = synth.make_verify("c1", seed=86, B=8, target_std=6.0)
    ks = [0, 20, 0, 5, 0, 100, 31999, 0]
    ps = [0.9, 1.0, 0.5, 0.8, 1.0, 0.99, 1.0, 0.3]
    _check(vin, np.linspace(0.5, 1.5, 8), ks, ps, top_k_max=32000, seed=87)


def test_invalid_parameters_fail_alone():
    vin = synth.make_verify("c4", seed=88, B=8, V=20000)
    Ts = [0.8, 0.0, -1.0, float("nan"), float("inf"), 0.8, 0.8, 1.0]
    ks = [64, 64, 0, 0, 0, 300, 64, 0]              # 300 > top_k_max
    ps = [1.0, 1.0, 1.0, 1.0, 1.0, 1.0, float("nan"), 0.9]
    g, o = _check(vin, Ts, ks, ps, top_k_max=128, seed=89)
    bad = [1, 2, 3, 4, 5, 6]
    assert all(g.num_accepted[b] == -1 and g.req_flags[b] & binding.ERR_PARAM for b in bad)
    assert g.num_accepted[0] >= 0 and g.num_accepted[7] >= 0
    assert g.err_word & binding.ERR_PARAM


def test_uniform_arrays_match_the_scalars():
    # the per-request path with every request alike decides as the scalar call does
    vin = _redraw(synth.make_verify("c4", seed=90, B=12, V=50000), [0.8] * 12, [64] * 12,
                  [0.9] * 12, 91)
    a = VerifyOnDevice(vin, top_k=64, top_p=0.9)
    a.run()
    ga = a.result()
    b = VerifyOnDevice(vin, temps=[vin.T] * 12, top_ks=[64] * 12, top_ps=[0.9] * 12, top_k_max=64)
    b.run()
    gb = b.result()
    # filtered rows run the same select and merge: bit-identical
    for f in ("num_accepted", "num_emitted", "out_tokens", "row_thr", "row_nkept", "row_sum",
              "p_y", "q_y"):
        assert np.array_equal(getattr(ga, f), getattr(gb, f)), f


@pytest.mark.parametrize("wl", ["c2", "c1"])
def test_uniform_temperature_arrays_match_the_scalar(wl):
    # temperatures alone take the plain statistics with each row's log2(e) / T: equal
    # temperatures give the scalar call's results bit for bit, debug values included
    vin = synth.make_verify(wl, seed=97, B=12, V=30000 if wl == "c2" else None)
    a = VerifyOnDevice(vin)
    a.run()
    ga = a.result()
    b = VerifyOnDevice(vin, temps=[vin.T] * vin.B)
    b.run()
    gb = b.result()
    for f in ("num_accepted", "num_emitted", "out_tokens", "row_max", "row_sum", "p_y", "q_y",
              "resid_mass", "picked_prob", "req_flags"):
        assert np.array_equal(getattr(ga, f), getattr(gb, f)), f


def test_full_size_sampled_per_request_temperature():
    vin = synth.make_verify("c2", seed=92)
    rng = np.random.default_rng(93)
    Ts = rng.uniform(0.3, 1.5, vin.B)
    ps = np.where(rng.random(vin.B) < 0.5, 0.9, 1.0)
    reqs = sorted(rng.choice(vin.B, size=12, replace=False).tolist())
    _check(vin, Ts, 0, ps, requests=reqs, seed=94)


@pytest.mark.parametrize("wl,temps_only", [("c4", False), ("c1", False), ("c4", True)])
def test_fused_cycle_equals_three_calls_per_request(wl, temps_only):
    vin = synth.make_verify(wl, seed=95, B=12, V=30000 if wl == "c4" else None, k=3,
                            **({"top_k": 0} if temps_only else {}))
    rec = synth.KVRecipe(L=2, H=2, D=8, prefix_lo=100, prefix_hi=300, share_group=3,
                         share_blocks=2)
    kv = synth.make_kv(wl, vin, seed=95, recipe=rec)
    rng = np.random.default_rng(96)
    Ts = rng.uniform(0.4, 1.4, vin.B).astype(np.float32)
    ks = rng.choice([0, 8, 64, 2000], vin.B).astype(np.int32)
    ps = rng.choice([1.0, 0.9, 0.5], vin.B).astype(np.float32)
    if temps_only:
        Ts[3] = -1.0                          # an invalid temperature fails its request alone
        ks, ps = None, None
    outs = []
    for mode in ("calls", "fused"):
        log(f"[params-fused] {wl} {mode}")
        g_kv = KVOnDevice(kv, vin.B)
        g_v = VerifyOnDevice(vin, temps=Ts, top_ks=ks, top_ps=ps, top_k_max=2000)
        if mode == "calls":
            g_kv.append(cu_new=g_v.cu + torch.arange(vin.B + 1, dtype=torch.int32,
                                                     device=g_v.cu.device))
            g_v.run()
            g_kv.rollback(g_v.num_acc, g_v.cu)
        else:
            dt = binding.SPECDEC_BF16 if vin.dtype == "bf16" else binding.SPECDEC_F32
            ws = torch.empty(binding.specdec_cycle_workspace_size(vin.B, vin.K, vin.V, dt, 0, 1.0,
                                                                  g_v.params),
                             dtype=torch.uint8, device=g_v.tgt.device)
            binding.specdec_cycle(g_kv.cache, g_kv.k_new, g_kv.v_new, g_v.tgt, g_v.dft,
                                  g_v.tokens, g_v.cu, g_v.u_acc, g_v.u_smp, max_k=vin.max_k,
                                  temperature=1.0, top_k=0, out_tokens=g_v.out_tokens,
                                  num_accepted=g_v.num_acc, num_emitted=g_v.num_emit,
                                  err_word=g_v.err, workspace=ws, debug=g_v.dbg,
                                  temperatures=g_v.temps, top_ks=g_v.top_ks, top_ps=g_v.top_ps,
                                  top_k_max=2000)
        outs.append((g_v.result(), g_kv.meta(), g_kv.pool.view(torch.int16).cpu().numpy()))
    a, b = outs
    for f in ("num_accepted", "num_emitted", "out_tokens", "err_word", "p_y", "q_y", "row_sum",
              "row_thr", "row_nkept", "resid_mass", "picked_prob", "req_flags"):
        assert np.array_equal(np.asarray(getattr(a[0], f)), np.asarray(getattr(b[0], f))), f
    for f in ("tables", "seq_lens", "refcount", "free_list", "free_count", "state"):
        assert np.array_equal(np.asarray(a[1][f]), np.asarray(b[1][f])), f
    assert np.array_equal(a[2], b[2])
    # and the decisions are the oracle's
    ok_, op_ = (0, 1.0) if temps_only else (ks, ps)
    o = oracle_verify(vin, T=Ts, top_k=ok_, top_p=op_, top_k_max=2000)
    rep = compare_verify(vin, a[0], o, T=Ts, top_k=ok_, top_p=op_)
    log(f"[params-fused]   {rep}")
    rep.check()
    o_kv = oracle_kv(kv)
    o_kv.append(kv.k_new, kv.v_new, kv.cu_new)
    o_kv.rollback(a[0].num_accepted, vin.cu_draft)
    errs = compare_kv_meta(o_kv, b[1], wl)
    assert not errs, "\n".join(errs)
