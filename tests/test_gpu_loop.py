"""Target and draft caches on the GPU over many speculative rounds ("Keep cache validity
aligned with the committed token history", paragraphs 1-2 and 5-6).

Each round, per request: the draft appends the states of its pending token(s) and
y_1 .. y_{k-1} (kv_paged_append); the target runs specdec_cycle (append of the pending
token and y_1 .. y_k, verification, rollback); kv_rollback_draft realigns the draft cache.
The emitted tokens extend the committed history. After every round both caches must hold
exactly the states of the committed history (a rejected state left valid would be
contamination), as much of it as each model has processed, the oracle's metadata bit for
bit, and every block accounted for (a leak).
"""

import numpy as np
import pytest
import torch

from gpu_harness import VerifyOnDevice, compare_kv_data, compare_kv_meta, dev, log
import oracle
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu

L, H, D, BS = 2, 2, 8, 16


def _state(model, b, pos, tok):
    """The K/V a model computes at position pos of request b for token tok (stand-in)."""
    r = np.random.default_rng([model, b, pos, tok])
    return r.integers(0, 0x7f00, size=(L, 2, H, D), dtype=np.uint16)


def _stack(model, b, pos0, toks):
    if not toks:
        return np.zeros((L, 2, 0, H, D), np.uint16)
    return np.stack([_state(model, b, pos0 + i, t) for i, t in enumerate(toks)], axis=2)


class Caches:
    """One paged cache on the device and the oracle's copy of it."""

    def __init__(self, B, NB, MBR, seed):
        d = dev()
        order = np.random.default_rng(seed).permutation(NB).astype(np.int32)
        self.pool = torch.empty((L, 2, NB, BS, H, D), dtype=torch.bfloat16, device=d)
        self.pool.view(torch.int16).fill_(0x7FAA)
        self.dev = binding.PagedKVCache(
            self.pool, torch.full((B, MBR), -1, dtype=torch.int32, device=d),
            torch.zeros(B, dtype=torch.int32, device=d),
            torch.zeros(NB, dtype=torch.int32, device=d), torch.from_numpy(order).to(d),
            torch.tensor([NB], dtype=torch.int32, device=d),
            torch.zeros(1, dtype=torch.int32, device=d))
        self.ora = oracle.PagedKV(L, H, D, BS, NB, np.full((B, MBR), -1), [0] * B, [0] * NB,
                                  list(order), NB, {})
        self.B = B

    def entries(self, stacks):
        """k / v [L][N][H][D] (host uint16 and device bf16) and cu for per-request stacks."""
        n = [s.shape[2] for s in stacks]
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        if cu[-1]:
            k = np.ascontiguousarray(np.concatenate([s[:, 0] for s in stacks], axis=1))
            v = np.ascontiguousarray(np.concatenate([s[:, 1] for s in stacks], axis=1))
        else:
            k = v = np.zeros((L, 0, H, D), np.uint16)
        to_dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev())
        return k, v, cu, to_dev(k), to_dev(v)

    def meta(self):
        torch.cuda.synchronize()
        c = self.dev
        return dict(tables=c.block_tables.cpu().numpy(), seq_lens=c.seq_lens.cpu().numpy(),
                    refcount=c.refcount.cpu().numpy(), free_list=c.free_list.cpu().numpy(),
                    free_count=int(c.free_count.item()), state=int(c.state.item()))


@pytest.mark.parametrize("seed,repeat", [(0, False), (1, False), (2, True)])
def test_target_and_draft_caches_over_rounds(seed, repeat):
    # repeat: every proposal of a round repeats the request's pending token id ("Keep cache
    # validity aligned with the committed token history", paragraph 6): the caches hold
    # one state per position, whatever the ids
    B, NB, MBR, V, rounds = 8, 600, 64, 64, 12
    rng = np.random.default_rng(200 + seed)
    tgt = Caches(B, NB, MBR, 300 + seed)
    dft = Caches(B, NB, MBR, 400 + seed)
    hist = [[int(rng.integers(V))] for _ in range(B)]      # one pending token per request
    for rnd in range(rounds):
        vin = synth.make_verify("c1", seed=1000 * seed + rnd, B=B, V=V, k_range=(0, 5))
        cu = [int(x) for x in vin.cu_draft]
        if repeat:
            for b in range(B):
                vin.draft_tokens[cu[b]:cu[b + 1]] = hist[b][-1]
        y = [[int(t) for t in vin.draft_tokens[cu[b]:cu[b + 1]]] for b in range(B)]
        log(f"[loop] seed {seed} round {rnd}: k_b = {[len(t) for t in y]}")
        # drafting: the draft processes its pending tokens, then y_1 .. y_{k-1}
        d0 = list(dft.ora.seq_lens)
        dk, dv, dcu, dk_d, dv_d = dft.entries(
            [_stack(1, b, d0[b], hist[b][d0[b]:] + y[b][:-1]) if y[b] else _stack(1, b, 0, [])
             for b in range(B)])
        ws = torch.empty(max(binding.kv_paged_append_workspace_size(B, int(dcu[-1])), 16),
                         dtype=torch.uint8, device=dev())
        binding.kv_paged_append(dft.dev, dk_d, dv_d, torch.from_numpy(dcu).to(dev()), ws)
        assert dft.ora.append(dk, dv, dcu) == 0
        # verification cycle of the target: pending token and y_1 .. y_k
        t0 = list(tgt.ora.seq_lens)
        tk, tv, tcu, tk_d, tv_d = tgt.entries(
            [_stack(0, b, t0[b], [hist[b][-1]] + y[b]) for b in range(B)])
        assert list(tcu) == [cu[b] + b for b in range(B + 1)]
        g = VerifyOnDevice(vin)
        wsc = torch.empty(binding.specdec_cycle_workspace_size(B, vin.K, V, binding.SPECDEC_F32, 0),
                          dtype=torch.uint8, device=dev())
        binding.specdec_cycle(tgt.dev, tk_d, tv_d, g.tgt, g.dft, g.tokens, g.cu, g.u_acc, g.u_smp,
                              max_k=vin.max_k, temperature=vin.T, top_k=0,
                              out_tokens=g.out_tokens, num_accepted=g.num_acc,
                              num_emitted=g.num_emit, err_word=g.err, workspace=wsc)
        binding.kv_rollback(dft.dev, g.num_acc, g.cu, draft=True)
        acc = g.num_acc.cpu().numpy()
        out = g.out_tokens.cpu().numpy()
        assert (acc >= 0).all() and int(g.err.item()) == 0
        # the oracle's caches take the same steps with the GPU's accepted counts
        assert tgt.ora.append(tk, tv, tcu) == 0
        assert tgt.ora.rollback(acc, cu) == 0
        assert dft.ora.rollback(acc, cu, draft=True) == 0
        for b in range(B):
            hist[b] += [int(t) for t in out[cu[b] + b: cu[b] + b + acc[b] + 1]]
        for c, name in ((tgt, "target"), (dft, "draft")):
            m = c.meta()
            errs = compare_kv_meta(c.ora, m, f"{name} round {rnd}") + compare_kv_data(c.ora, c.pool)
            assert not errs, "\n".join(errs)
            assert m["state"] == 0
            c.ora.check_invariants()
        for b in range(B):
            n = len(hist[b])
            assert tgt.ora.seq_lens[b] == n - 1
            assert np.array_equal(tgt.ora.logical_view(b), _stack(0, b, 0, hist[b][:n - 1]))
            keep = dft.ora.seq_lens[b]
            pending_before = t0[b] + 1 - d0[b]
            k = len(y[b])
            assert keep == (d0[b] + pending_before + min(int(acc[b]), k - 1) if k else d0[b])
            assert np.array_equal(dft.ora.logical_view(b), _stack(1, b, 0, hist[b][:keep]))
