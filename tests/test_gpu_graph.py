"""The fused cycle captured once in a HIP graph and replayed: each replay is the next cycle
(the launches read their sizes and pointers from arguments or device memory), so replays
equal eager cycles on a twin cache bit for bit, with the program's own eager work and
synchronizations between the replays. The library records no memset or allocation."""

import numpy as np
import pytest
import torch

from gpu_harness import KVOnDevice, VerifyOnDevice, log
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu


def _cycle(g_kv, g_v, vin, ws, early=False):
    binding.specdec_cycle(g_kv.cache, g_kv.k_new, g_kv.v_new, g_v.tgt, g_v.dft, g_v.tokens,
                          g_v.cu, g_v.u_acc, g_v.u_smp, max_k=vin.max_k, temperature=vin.T,
                          top_k=vin.top_k, out_tokens=g_v.out_tokens, num_accepted=g_v.num_acc,
                          num_emitted=g_v.num_emit, err_word=g_v.err, workspace=ws,
                          debug=g_v.dbg, top_p=g_v.top_p, early_exit=early)


@pytest.mark.parametrize("wl,top_p,early", [("c4", 1.0, False), ("c2", 0.9, False),
                                            ("c1", 1.0, False), ("c2", 1.0, True),
                                            ("c1", 1.0, True)])
def test_graph_replays_equal_eager_cycles(wl, top_p, early):
    # early: the early-exit cycle (its liveness flags live in the workspace and are
    # rewritten by every replay's first launch)
    vin = synth.make_verify(wl, seed=140, B=12, V=20000 if wl != "c1" else 4000, k=4)
    rec = synth.KVRecipe(L=2, H=2, D=8, prefix_lo=40, prefix_hi=300, share_group=3,
                         share_blocks=2)
    kv = synth.make_kv(wl, vin, seed=140, recipe=rec, cycles=8)
    dt = binding.SPECDEC_BF16 if vin.dtype == "bf16" else binding.SPECDEC_F32
    nbytes = binding.specdec_cycle_workspace_size(vin.B, vin.K, vin.V, dt, vin.top_k, top_p)
    eager = (KVOnDevice(kv, vin.B), VerifyOnDevice(vin, top_p=top_p))
    graph = (KVOnDevice(kv, vin.B), VerifyOnDevice(vin, top_p=top_p))
    ws_e = torch.empty(nbytes, dtype=torch.uint8, device=eager[1].tgt.device)
    ws_g = torch.empty(nbytes, dtype=torch.uint8, device=eager[1].tgt.device)
    log(f"[graph] {wl} top_p={top_p} early_exit={early}: capture")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _cycle(*graph, vin, ws_g, early)
    torch.cuda.synchronize()
    x = torch.randn(256, 256, device=eager[1].tgt.device)
    for it in range(4):
        _cycle(*eager, vin, ws_e, early)
        g.replay()
        torch.cuda.synchronize()
        x = (x @ x.T).tanh()              # the program's own work between replays
        torch.cuda.synchronize()
        a, b = eager[1].result(), graph[1].result()
        for f in ("num_accepted", "num_emitted", "out_tokens", "err_word", "p_y", "q_y",
                  "row_sum", "resid_mass", "picked_prob", "req_flags"):
            assert np.array_equal(np.asarray(getattr(a, f)), np.asarray(getattr(b, f)),
                                  equal_nan=True), (it, f)
        ma, mb = eager[0].meta(), graph[0].meta()
        for f in ("tables", "seq_lens", "refcount", "free_list", "free_count", "state"):
            assert np.array_equal(np.asarray(ma[f]), np.asarray(mb[f])), (it, f)
        assert torch.equal(eager[0].pool.view(torch.int16), graph[0].pool.view(torch.int16)), it
        log(f"[graph]   cycle {it}: accepted {int(a.num_accepted.sum())}, "
            f"seq_lens sum {int(ma['seq_lens'].sum())}")
    assert int(ma["seq_lens"].sum()) > int(kv.seq_lens.sum())   # the cache did grow
