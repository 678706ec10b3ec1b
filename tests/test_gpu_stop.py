"""GPU stopping at an accepted end-of-sequence token or an output cap, against the oracle
("Keep cache validity aligned with the committed token history", paragraph 6: EOS and
output caps among the cases to test). Stopped requests emit the cut proposals and draw
nothing; the cycle's cache keeps the pending token and the emitted proposals."""

import numpy as np
import pytest
import torch

from gpu_harness import (KVOnDevice, VerifyOnDevice, compare_kv_meta, compare_verify, log,
                         oracle_kv, oracle_verify)
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu


def _stops(vin, seed):
    """EOS tokens and caps that cut some requests inside their accepted proposals."""
    base = oracle_verify(vin)
    rng = np.random.default_rng(seed)
    eos = np.full(vin.B, -1, dtype=np.int32)
    cap = np.zeros(vin.B, dtype=np.int32)
    for b in range(vin.B):
        a = int(base.num_accepted[b])
        if a < 0:
            continue
        em = base.requests[b].emitted
        if b % 3 == 0 and a >= 1:
            eos[b] = em[int(rng.integers(0, a))]
        elif b % 3 == 1:
            cap[b] = int(rng.integers(1, a + 3))
        else:
            eos[b] = em[a]
    return eos, cap


@pytest.mark.parametrize("wl,over", [("c1", dict(classes=((1.0, "noise", 0.1),))),
                                     ("c4", dict(V=30000, k=6, classes=((1.0, "noise", 0.2),)))])
def test_stopping_matches_oracle(wl, over):
    vin = synth.make_verify(wl, seed=130, B=16, **over)
    eos, cap = _stops(vin, 131)
    v = VerifyOnDevice(vin, eos=eos, max_emit=cap)
    v.run()
    g = v.result()
    o = oracle_verify(vin, eos=eos, max_emit=cap)
    rep = compare_verify(vin, g, o, eos=eos, max_emit=cap)
    log(f"[stop] {wl}: {rep} stopped={rep.stopped}")
    rep.check()
    assert rep.stopped >= 3


def test_stopping_in_the_fused_cycle():
    vin = synth.make_verify("c4", seed=132, B=12, V=20000, k=5, classes=((1.0, "noise", 0.2),))
    eos, cap = _stops(vin, 133)
    rec = synth.KVRecipe(L=2, H=2, D=8, prefix_lo=30, prefix_hi=200)
    kv = synth.make_kv("c4", vin, seed=132, recipe=rec)
    outs = []
    for mode in ("calls", "fused"):
        g_kv = KVOnDevice(kv, vin.B)
        g_v = VerifyOnDevice(vin, eos=eos, max_emit=cap)
        if mode == "calls":
            g_kv.append()
            g_v.run()
            g_kv.rollback(g_v.num_acc, g_v.cu)
        else:
            dt = binding.SPECDEC_BF16
            ws = torch.empty(binding.specdec_cycle_workspace_size(vin.B, vin.K, vin.V, dt,
                                                                  vin.top_k, 1.0, g_v.params),
                             dtype=torch.uint8, device=g_v.tgt.device)
            binding.specdec_cycle(g_kv.cache, g_kv.k_new, g_kv.v_new, g_v.tgt, g_v.dft, g_v.tokens,
                                  g_v.cu, g_v.u_acc, g_v.u_smp, max_k=vin.max_k,
                                  temperature=vin.T, top_k=vin.top_k, out_tokens=g_v.out_tokens,
                                  num_accepted=g_v.num_acc, num_emitted=g_v.num_emit,
                                  err_word=g_v.err, workspace=ws, debug=g_v.dbg,
                                  eos_tokens=g_v.eos, max_emit=g_v.max_emit)
        outs.append((g_v.result(), g_kv.meta()))
    (ga, ma), (gb, mb) = outs
    for f in ("num_accepted", "num_emitted", "out_tokens", "req_flags"):
        assert np.array_equal(getattr(ga, f), getattr(gb, f)), f
    for f in ("tables", "seq_lens", "refcount", "free_list", "free_count", "state"):
        assert np.array_equal(np.asarray(ma[f]), np.asarray(mb[f])), f
    o = oracle_verify(vin, eos=eos, max_emit=cap)
    rep = compare_verify(vin, gb, o, eos=eos, max_emit=cap)
    rep.check()
    o_kv = oracle_kv(kv)
    o_kv.append(kv.k_new, kv.v_new, kv.cu_new)
    o_kv.rollback(gb.num_accepted, vin.cu_draft)
    errs = compare_kv_meta(o_kv, mb, "stop")
    assert not errs, "\n".join(errs)
    for b in range(vin.B):
        assert mb["seq_lens"][b] == kv.seq_lens[b] + 1 + gb.num_accepted[b]
