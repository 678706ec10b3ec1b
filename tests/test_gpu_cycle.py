"""One full speculative cycle per workload on the GPU, stream-ordered with no host sync
between the calls: kv_paged_append -> specdec_verify -> kv_rollback (rollback consumes the
device num_accepted). Checked against the oracle on every request: decisions and tokens
(flagged-margin rule), then the oracle's append / rollback with the same accepted counts,
bit for bit on metadata and K/V."""

import numpy as np
import pytest

from gpu_harness import (KVOnDevice, VerifyOnDevice, compare_kv_data, compare_kv_meta,
                         compare_verify, log, oracle_kv, oracle_verify)
from rejection_sampling_verify_specdec_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", ["c1", "c2", "c3", "c4"])
def test_cycle(wl):
    vin = synth.make_verify(wl, seed=0)
    log(f"[cycle] {wl}: B={vin.B} K={vin.K} V={vin.V}; oracle verify")
    o = oracle_verify(vin, keep_probs=False)
    kv = synth.make_kv(wl, vin, seed=0, a_hint=o.num_accepted)
    log(f"[cycle] {wl}: NB={kv.num_blocks} L={kv.L}; GPU cycle")
    g_kv = KVOnDevice(kv, vin.B)
    g_v = VerifyOnDevice(vin)
    g_kv.append()
    g_v.run()
    g_kv.rollback(g_v.num_acc, g_v.cu)
    g = g_v.result()
    rep = compare_verify(vin, g, o)
    log(f"[cycle] {wl}: {rep}")
    assert not rep.errors, "\n".join(rep.errors)
    # the oracle cache follows the GPU's accepted counts (identical unless flagged)
    o_kv = oracle_kv(kv)
    o_kv.append(kv.k_new, kv.v_new, kv.cu_new)
    o_kv.rollback(g.num_accepted, vin.cu_draft)
    errs = compare_kv_meta(o_kv, g_kv.meta(), wl) + compare_kv_data(o_kv, g_kv.pool)
    assert not errs, "\n".join(errs)
    o_kv.check_invariants()
    if kv.block_size and wl == "c3":
        # rejected requests end exactly on a block boundary
        rej = [b for b in range(vin.B) if 0 <= g.num_accepted[b] < vin.k_b[b]]
        assert all(o_kv.seq_lens[b] % kv.block_size == 0 for b in rej)
