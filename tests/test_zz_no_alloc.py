"""specdec_cycle_static (the cycle over the library's static scratch array, for callers that
cannot allocate) against specdec_cycle with a caller workspace, on twin inputs and caches:
accepted counts, emitted tokens, error word, request flags, debug values, cache metadata
and pool bits equal bit for bit, over two calls in a row, the second with a smaller batch
and vocabulary; a call larger than the array is refused before anything is enqueued."""

import numpy as np
import pytest
import torch

from gpu_harness import KVOnDevice, VerifyOnDevice, log
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu


def _cycle(vin, kv, static):
    g_kv = KVOnDevice(kv, vin.B)
    g_v = VerifyOnDevice(vin)
    kw = dict(max_k=vin.max_k, temperature=vin.T, top_k=vin.top_k, out_tokens=g_v.out_tokens,
              num_accepted=g_v.num_acc, num_emitted=g_v.num_emit, err_word=g_v.err,
              debug=g_v.dbg)
    args = (g_kv.cache, g_kv.k_new, g_kv.v_new, g_v.tgt, g_v.dft, g_v.tokens, g_v.cu, g_v.u_acc,
            g_v.u_smp)
    if static:
        binding.specdec_cycle_static(*args, **kw)
    else:
        dt = binding.SPECDEC_BF16 if vin.dtype == "bf16" else binding.SPECDEC_F32
        ws = torch.full((binding.specdec_cycle_workspace_size(vin.B, vin.K, vin.V, dt,
                                                              vin.top_k),),
                        0x3C, dtype=torch.uint8, device=g_v.tgt.device)
        binding.specdec_cycle(*args, workspace=ws, **kw)
    r = g_v.result()
    return r, g_kv.meta(), g_kv.pool.view(torch.int16).cpu().numpy()


def _same(vin, kv, what):
    log(f"[no-alloc] {what}: B={vin.B} K={vin.K} V={vin.V} {vin.dtype}")
    (a, am, ap), (b, bm, bp) = _cycle(vin, kv, False), _cycle(vin, kv, True)
    for name in ("num_accepted", "num_emitted", "out_tokens", "err_word", "p_y", "q_y",
                 "row_max", "row_sum", "resid_mass", "picked_prob", "req_flags"):
        assert np.array_equal(np.asarray(getattr(a, name)), np.asarray(getattr(b, name)),
                              equal_nan=True), name
    for name in ("tables", "seq_lens", "refcount", "free_list", "free_count", "state"):
        assert np.array_equal(np.asarray(am[name]), np.asarray(bm[name])), name
    assert np.array_equal(ap, bp), "pool bits"
    log(f"[no-alloc]   accepted {int(a.num_accepted[a.num_accepted >= 0].sum())}, "
        f"err {a.err_word:#x}: identical")


def test_static_scratch_cycle_equals_the_workspace_cycle():
    rec = synth.KVRecipe(L=2, H=2, D=8, prefix_lo=40, prefix_hi=300, share_group=3,
                         share_blocks=2)
    vin = synth.make_verify("c2", seed=170, B=40, V=20000)
    _same(vin, synth.make_kv("c2", vin, seed=170, recipe=rec), "first call")
    small = synth.make_verify("c1", seed=171, B=7, V=5003, k_range=(0, 6), k=6)
    _same(small, synth.make_kv("c1", small, seed=171, recipe=rec), "second call, smaller")


def test_call_larger_than_the_scratch_is_refused():
    # top-k candidate lists of the full c4 batch need ~73 MB: refused, outputs untouched
    vin = synth.make_verify("c4", seed=172, V=128256)
    dt = binding.SPECDEC_BF16
    need = binding.specdec_cycle_workspace_size(vin.B, vin.K, vin.V, dt, vin.top_k)
    assert need > binding.STATIC_SCRATCH_BYTES
    rec = synth.KVRecipe(L=1, H=2, D=8, prefix_lo=40, prefix_hi=300)
    g_kv = KVOnDevice(synth.make_kv("c4", vin, seed=172, recipe=rec), vin.B)
    g_v = VerifyOnDevice(vin)
    with pytest.raises(binding.SpecdecError) as e:
        binding.specdec_cycle_static(g_kv.cache, g_kv.k_new, g_kv.v_new, g_v.tgt, g_v.dft,
                                     g_v.tokens, g_v.cu, g_v.u_acc, g_v.u_smp, max_k=vin.max_k,
                                     temperature=vin.T, top_k=vin.top_k,
                                     out_tokens=g_v.out_tokens, num_accepted=g_v.num_acc,
                                     num_emitted=g_v.num_emit, err_word=g_v.err)
    assert e.value.status == binding.SPECDEC_ESCRATCH
    torch.cuda.synchronize()
    assert (g_v.num_acc.cpu().numpy() == -9).all()
