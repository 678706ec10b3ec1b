"""GPU verification of draft trees and the cache step that keeps the accepted path, against
the oracle ("Speculative decoding: accelerate LLM generation without changing its
answers", sections 2-3, with the residual applied sibling after sibling; "Keep cache
validity aligned with the committed token history", paragraphs 3 and 6).

Rule: accepted paths, emitted tokens and flags equal the oracle's, except requests whose
walk met a decision within 1e-6 of its threshold (|u - P/Q| of a tried node, or the draw's
distance to a CDF edge as a fraction of W), or read a row whose nucleus (top-p) decision
lies within 2e-6 of top_p, and requests whose walk formed a residual mass below
4 * 2^-20: the device's residual chain is built from fp32 exponentials and clamps a
mass at or below 2^-20 to zero (drawing from the distribution the child was tested
against), so near that clamp its fallback decision is rounding's. Both classes are counted
and checked for validity only: the path is a root-to-node chain whose tokens were emitted,
followed by one drawn token with positive target probability at the path's end; their
mismatches stay within a bound. Cache metadata and K/V bits equal the oracle's after the
oracle applies the GPU's accepted paths.
"""

import numpy as np
import pytest
import torch

from gpu_harness import (NUCLEUS_MARGIN, _nucleus_floor, compare_kv_data, compare_kv_meta, dev,
                         log, pool_tensor)
import oracle
from rejection_sampling_verify_specdec_amd import binding, synth

pytestmark = pytest.mark.gpu

MARGIN = 1e-6


def _t(x, d):
    return torch.from_numpy(np.ascontiguousarray(x)).to(d)


def _logits(x, dtype, d):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(d)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(d)


class TreeOnDevice:
    def __init__(self, tin, team: int = 0, ws_fill: int = 0, top_k: int = 0, top_p: float = 1.0,
                 temps=None, top_ks=None, top_ps=None, top_k_max=None):
        d = dev()
        self.team = team
        self.top_k, self.top_p = top_k, top_p
        opt = lambda x: None if x is None else _t(np.asarray(x), d)
        self.temps, self.top_ks, self.top_ps = opt(temps), opt(top_ks), opt(top_ps)
        self.top_k_max = top_k_max
        self.tin = tin
        self.tgt = _logits(tin.target, tin.dtype, d)
        self.dft = _logits(tin.draft, tin.dtype, d)
        self.tokens, self.parent = _t(tin.tokens, d), _t(tin.parent, d)
        self.cu = _t(tin.cu_nodes, d)
        self.u_acc, self.u_smp = _t(tin.u_accept, d), _t(tin.u_sample, d)
        B, N = tin.B, tin.N
        self.out = torch.full((N + B,), -7, dtype=torch.int32, device=d)
        self.nodes = torch.full((N,), -7, dtype=torch.int32, device=d)
        self.num_acc = torch.full((B,), -9, dtype=torch.int32, device=d)
        self.num_emit = torch.full((B,), -9, dtype=torch.int32, device=d)
        self.err = torch.zeros(1, dtype=torch.int32, device=d)
        self.flags = torch.full((B,), -1, dtype=torch.int32, device=d)
        # the call resets what it needs: start from arbitrary contents
        dt = binding.SPECDEC_BF16 if tin.dtype == "bf16" else binding.SPECDEC_F32
        prm = binding._params(B, d, self.temps, self.top_ks, self.top_ps, top_k_max)
        self.ws = torch.full((binding.specdec_tree_verify_workspace_size(B, N, tin.V, dt, top_k,
                                                                         top_p, prm),),
                             ws_fill, dtype=torch.uint8, device=d)

    def run(self):
        binding.specdec_tree_verify(self.tgt, self.dft, self.tokens, self.parent, self.cu,
                                    self.u_acc, self.u_smp, max_nodes=self.tin.max_nodes,
                                    temperature=self.tin.T, out_tokens=self.out,
                                    accepted_nodes=self.nodes, num_accepted=self.num_acc,
                                    num_emitted=self.num_emit, err_word=self.err,
                                    workspace=self.ws, req_flags=self.flags, team=self.team,
                                    top_k=self.top_k, top_p=self.top_p, temperatures=self.temps,
                                    top_ks=self.top_ks, top_ps=self.top_ps,
                                    top_k_max=self.top_k_max)
        torch.cuda.synchronize()
        c = lambda x: x.cpu().numpy()
        return dict(a=c(self.num_acc), n=c(self.num_emit), out=c(self.out), nodes=c(self.nodes),
                    err=int(self.err.item()), flags=c(self.flags))


TREE_CLAMP = 2.0 ** -20


def _flagged(res):
    if res is None or res.res is None:
        return False
    r = res.res
    return any(m < MARGIN for m in r.accept_margin) or (r.sample_margin is not None and
                                                        r.sample_margin < MARGIN)


def _nucleus_close(res):
    return res is not None and res.nucleus_margin < NUCLEUS_MARGIN


def _near_clamp(res):
    """The walk formed a residual mass within a factor of 4 of the device's clamp."""
    return res is not None and res.res is not None and \
        any(0 < float(W) < 4 * TREE_CLAMP for W in res.res.resid_W)


def _valid(tin, g, b, ga, top_k=0, top_p=1.0, T=None):
    """A valid walk result: a root-to-node chain, its tokens emitted in order, one more
    token drawn with positive target probability at the position the path ends (inside
    the row's top-k set, and its nucleus decided either way)."""
    errs = []
    lo, hi = int(tin.cu_nodes[b]), int(tin.cu_nodes[b + 1])
    path = [int(j) for j in g["nodes"][lo: lo + ga]]
    got = [int(x) for x in g["out"][lo + b: lo + b + ga + 1]]
    par = tin.parent[lo:hi]
    prev = -1
    for j in path:
        if not 0 <= j < hi - lo or par[j] != prev:
            errs.append(f"req {b}: path {path} is not a chain")
            return errs
        prev = j
    if got[:ga] != [int(tin.tokens[lo + j]) for j in path]:
        errs.append(f"req {b}: emitted {got[:ga]} are not the path's tokens")
    if int(g["n"][b]) != ga + 1:
        errs.append(f"req {b}: num_emitted {g['n'][b]}")
    pos = 0 if not path else path[-1] + 1
    z = oracle.verify._decode_rows(tin.target[lo + b + pos: lo + b + pos + 1], tin.dtype)[0]
    x = got[ga] if len(got) > ga else -1
    floor = _nucleus_floor(z, tin.T if T is None else T, top_k, top_p) \
        if (0 < top_k < tin.V or 0 < top_p < 1) else -np.inf
    if not (0 <= x < tin.V and z[x] > -np.inf and z[x] >= floor):
        errs.append(f"req {b}: drawn token {x} has no target probability")
    return errs


def compare_tree(tin, g, o, top_k=0, top_p=1.0, T=None):
    """errors, flagged requests (margin, nucleus or clamp), flagged mismatches; the caller
    asserts that there are no errors (the bound on mismatches is one of them). T, top_k,
    top_p: scalars or per-request arrays."""
    flagged = mism = decisions = 0
    errs = []
    per = lambda x, f: [f(v) for v in np.broadcast_to(np.asarray(x), (tin.B,))]
    Ts = per(tin.T if T is None else T, lambda v: float(np.float32(v)))
    ks = per(top_k, int)
    ps = per(top_p, lambda v: float(np.float32(v)))
    for b in range(tin.B):
        oa, ga = int(o.num_accepted[b]), int(g["a"][b])
        r = o.requests[b]
        fl = _flagged(r) or _near_clamp(r) or _nucleus_close(r)
        if int(o.err[b]) != int(g["flags"][b]) and not fl:
            errs.append(f"req {b}: flags oracle {o.err[b]} gpu {g['flags'][b]}")
        if oa < 0 or ga < 0:
            if oa != ga:
                errs.append(f"req {b}: error status oracle {oa} gpu {ga}")
            continue
        lo = int(tin.cu_nodes[b])
        decisions += len(r.res.tried) + 1
        got = list(g["out"][lo + b: lo + b + ga + 1])
        path = list(g["nodes"][lo: lo + ga])
        flagged += fl
        errs += _valid(tin, g, b, ga, ks[b], ps[b], Ts[b])
        if oa != ga or got != r.emitted or path != r.path:
            if fl:
                mism += 1
                continue
            errs.append(f"req {b}: path {path} vs {r.path}, tokens {got} vs {r.emitted}")
    if mism > 2 + decisions // 1000:
        errs.append(f"{mism} flagged mismatches over the bound ({decisions} decisions)")
    return errs, flagged, mism


def _check(tin, top_k=0, top_p=1.0, team=0, temps=None, top_ks=None, top_ps=None,
           top_k_max=None):
    log(f"[tree] B={tin.B} N={tin.N} V={tin.V} {tin.dtype} T={tin.T} top_k={top_k} "
        f"top_p={top_p} team={team} per-request={temps is not None or top_ks is not None or top_ps is not None}")
    g = TreeOnDevice(tin, top_k=top_k, top_p=top_p, team=team, temps=temps, top_ks=top_ks,
                     top_ps=top_ps, top_k_max=top_k_max).run()
    T = tin.T if temps is None else temps
    k = top_k if top_ks is None else top_ks
    p = top_p if top_ps is None else top_ps
    o = oracle.tree_verify_batch(tin.target, tin.draft, tin.tokens, tin.parent, tin.cu_nodes,
                                 tin.u_accept, tin.u_sample, T, tin.max_nodes, tin.dtype,
                                 top_k=k, top_p=p, top_k_max=top_k_max)
    errs, fl, mism = compare_tree(tin, g, o, k, p, T)
    log(f"[tree]   accepted mean {np.mean(g['a'][g['a'] >= 0]) if (g['a'] >= 0).any() else 0:.2f}, "
        f"flagged {fl}, flagged mismatches {mism}")
    assert not errs, "\n".join(errs[:20])
    return g, o


@pytest.mark.parametrize("dtype,V", [("bf16", 128256), ("f32", 32000), ("bf16", 4001)])
def test_tree_matches_oracle(dtype, V):
    _check(synth.make_tree(seed=110, B=12, V=V, dtype=dtype, n_range=(1, 20)))


def test_tree_wide_and_deep():
    # wide: every node a child of the root; deep: chains (branch 0)
    _check(synth.make_tree(seed=111, B=6, V=20000, n_range=(30, 64), branch=1.0))
    _check(synth.make_tree(seed=112, B=6, V=20000, n_range=(30, 64), branch=0.0))


def test_tree_close_drafts_accept_deep():
    _check(synth.make_tree(seed=113, B=8, V=50000, n_range=(8, 24), noise_std=0.2))


def test_tree_branch_switch():
    # first child of the root has p = 0 (its logit -inf in the target row): always
    # rejected; the walk must continue with the second child against the residual
    tin = synth.make_tree(seed=114, B=4, V=1000, dtype="f32", n_range=(3, 3), branch=0.0,
                          noise_std=0.1)
    for b in range(tin.B):
        lo = int(tin.cu_nodes[b])
        tin.parent[lo: lo + 3] = [-1, -1, 1]
        tin.target[lo + b, tin.tokens[lo]] = -np.inf
        tin.tokens[lo + 1] = int(np.argmax(tin.target[lo + b]))
    g, o = _check(tin)
    assert all(1 in o.requests[b].res.tried for b in range(tin.B))


def test_tree_errors():
    tin = synth.make_tree(seed=115, B=6, V=3000, dtype="f32", n_range=(2, 5))
    cu = tin.cu_nodes
    tin.parent[cu[1] + 1] = 5                        # forward parent
    tin.tokens[cu[2]] = 3000                         # token out of range
    tin.u_accept[cu[3]] = 1.0                        # bad uniform
    tin.target[cu[4] + 4, 7] = np.nan                # NaN in the root row
    g, o = _check(tin)
    assert g["a"][0] >= 0 and g["a"][5] >= 0
    assert g["flags"][1] & binding.ERR_TREE and g["flags"][2] & binding.ERR_TOKEN
    assert g["flags"][3] & binding.ERR_UNIFORM and g["flags"][4] & binding.ERR_NONFINITE
    assert all(g["a"][b] == -1 for b in (1, 2, 3, 4))


def test_tree_too_many_nodes_and_empty_trees():
    tin = synth.make_tree(seed=117, B=5, V=2000, dtype="f32", n_range=(0, 6), max_nodes=4)
    assert tin.N <= tin.B * tin.max_nodes
    g, o = _check(tin)
    for b in range(tin.B):
        n = int(tin.cu_nodes[b + 1] - tin.cu_nodes[b])
        if n > 4:
            assert g["flags"][b] & binding.ERR_K and g["a"][b] == -1
        if n == 0:
            assert g["a"][b] == 0 and g["n"][b] == 1


def test_tree_deterministic():
    tin = synth.make_tree(seed=117, B=8, V=60000, n_range=(4, 16))
    outs = [TreeOnDevice(tin).run() for _ in range(3)]
    for o in outs[1:]:
        assert all(np.array_equal(outs[0][k], o[k]) for k in ("a", "out", "nodes", "flags"))


@pytest.mark.parametrize("dtype,V,top_k,top_p,std", [
    ("bf16", 128256, 64, 1.0, 3.0),       # top-k 64, as the linear top-k workload (listed)
    ("bf16", 128256, 0, 0.9, 3.0),        # top-p alone
    ("bf16", 128256, 0, 0.99, 1.0),       # a nucleus too large to list: full-row passes
    ("f32", 32000, 50, 0.9, 3.0),         # top-k, then top-p inside it (fp32: never listed)
    ("bf16", 20000, 2000, 1.0, 3.0),      # top-k past the chunk select's limit: generic
    ("bf16", 4001, 16, 0.95, 3.0),        # rows that are not whole 16-byte vectors
])
def test_tree_with_transforms(dtype, V, top_k, top_p, std):
    # the transform applies alike to every target and draft row the walk reads; the nodes
    # are drawn within the draft rows' top-k set. bf16 target rows whose kept tokens fit the
    # list are walked over the list alone, the others (and fp32) with masked full-row passes
    _check(synth.make_tree(seed=130, B=10, V=V, dtype=dtype, n_range=(1, 20), noise_std=0.5,
                           target_std=std, top_k=top_k), top_k, top_p)


def test_tree_transforms_with_ties_and_bad_rows():
    # bf16 rows with a block of equal logits at the top-k boundary (ties are kept), and
    # NaN planted in one request's root target row (the walk reads it: an error) and in
    # another's unvisited leaf draft row (never read: no error)
    tin = synth.make_tree(seed=133, B=12, V=30000, dtype="bf16", n_range=(2, 10),
                          noise_std=0.5, top_k=32)
    z = synth.bf16_bits_to_f32(tin.target)
    for r in range(tin.N + tin.B):
        top = np.argsort(z[r])[::-1]
        z[r, top[28:40]] = z[r, top[28]]          # 12 equal values across the 32nd place
    tin.target[:] = synth.f32_to_bf16_bits(z)
    lo1 = int(tin.cu_nodes[1])
    tin.target[lo1 + 1, 5] = 0x7fc0               # NaN in request 1's root target row
    lo2, hi2 = int(tin.cu_nodes[2]), int(tin.cu_nodes[3])
    leaf = max(j for j in range(hi2 - lo2) if j not in set(tin.parent[lo2:hi2]))
    tin.draft[lo2 + 2 + 1 + leaf, 7] = 0x7fc0     # NaN in a leaf's draft row (not read)
    g, o = _check(tin, 32, 1.0)
    assert g["flags"][1] & binding.ERR_NONFINITE and g["a"][1] == -1
    assert g["a"][2] >= 0


@pytest.mark.parametrize("top_k,top_p", [(30000, 1.0), (0, 0.0), (0, 1.0)])
def test_tree_transforms_that_are_off(top_k, top_p):
    # top_k >= V, top_p <= 0 or >= 1: no filter, the same outputs as temperature alone
    tin = synth.make_tree(seed=134, B=6, V=30000, dtype="bf16", n_range=(2, 12))
    ref = TreeOnDevice(tin).run()
    g = TreeOnDevice(tin, top_k=top_k, top_p=top_p).run()
    for key in ("a", "n", "out", "nodes", "flags"):
        assert np.array_equal(g[key], ref[key]), key


@pytest.mark.parametrize("dtype,V,step", [("f32", 3000, 0.01), ("bf16", 200, 0.25)])
@pytest.mark.parametrize("top_k,top_p", [(1, 1.0), (0, 1e-6)])
def test_tree_point_mass_transform_is_greedy(top_k, top_p, dtype, V, step):
    # top-k 1 (or a one-token nucleus) makes p and q point masses: the walk follows the
    # first child carrying the target row's argmax and emits that argmax where no child
    # does; distinct logits (exact in bf16 at V = 200), the draft's argmax never the
    # target's
    tin = synth.make_tree(seed=131, B=16, V=V, dtype=dtype, n_range=(0, 12), branch=0.6)
    rng = np.random.default_rng(5)
    R = tin.N + tin.B
    tz = np.stack([rng.permutation(V) for _ in range(R)]).astype(np.float32) * np.float32(step)
    dz = np.stack([rng.permutation(V) for _ in range(R)]).astype(np.float32) * np.float32(step)
    at = np.argmax(tz, axis=1)
    clash = np.argmax(dz, axis=1) == at
    dz[clash] = np.roll(dz[clash], 1, axis=1)
    if dtype == "bf16":
        tin.target[:] = synth.f32_to_bf16_bits(tz)
        tin.draft[:] = synth.f32_to_bf16_bits(dz)
        assert np.array_equal(synth.bf16_bits_to_f32(tin.target), tz)
    else:
        tin.target[:] = tz
        tin.draft[:] = dz
    for b in range(tin.B):
        lo, hi = int(tin.cu_nodes[b]), int(tin.cu_nodes[b + 1])
        for j in range(hi - lo):
            if rng.random() < 0.5:
                tin.tokens[lo + j] = at[lo + b + int(tin.parent[lo + j]) + 1]
    g, o = _check(tin, top_k, top_p)
    for b in range(tin.B):
        lo, hi = int(tin.cu_nodes[b]), int(tin.cu_nodes[b + 1])
        kids = oracle.tree.children_of([int(x) for x in tin.parent[lo:hi]])
        v, want = 0, []
        while True:
            a = int(at[lo + b + v])
            want.append(a)
            nxt = next((j for j in kids[v] if int(tin.tokens[lo + j]) == a), None)
            if nxt is None:
                break
            v = nxt + 1
        got = [int(x) for x in g["out"][lo + b: lo + b + int(g["n"][b])]]
        assert got == want, (b, got, want)


@pytest.mark.parametrize("top_k,top_p", [(64, 1.0), (0, 0.9)])
def test_team_sizes_with_transforms(top_k, top_p):
    tin = synth.make_tree(seed=132, B=6, V=128256, dtype="bf16", n_range=(5, 30),
                          noise_std=0.5, top_k=top_k)
    ref, _ = _check(tin, top_k, top_p, team=1)
    for team in (2, 7, 16):
        log(f"[tree-team]   team {team}, top_k {top_k}, top_p {top_p}")
        g = TreeOnDevice(tin, team=team, ws_fill=0xCD, top_k=top_k, top_p=top_p).run()
        for key in ("a", "n", "out", "nodes", "flags"):
            assert np.array_equal(g[key], ref[key]), (team, key)


@pytest.mark.parametrize("dtype,V", [("bf16", 128256), ("f32", 32000)])
def test_tree_per_request_transforms(dtype, V):
    # per-request temperature, top-k and top-p (each request its own transform on its p and
    # q rows), with an invalid temperature and a NaN top_p failing their requests alone
    tin = synth.make_tree(seed=135, B=14, V=V, dtype=dtype, n_range=(1, 16), noise_std=0.5)
    r = np.random.default_rng(9)
    temps = r.choice([0.5, 0.8, 1.2], tin.B).astype(np.float32)
    ks = r.choice([0, 8, 64, V], tin.B).astype(np.int32)
    ps = r.choice([1.0, 0.9, 0.5], tin.B).astype(np.float32)
    temps[3] = 0.0
    ps[7] = np.nan
    g, o = _check(tin, temps=temps, top_ks=ks, top_ps=ps, top_k_max=64)
    assert g["flags"][3] & binding.ERR_PARAM and g["flags"][7] & binding.ERR_PARAM
    assert g["a"][3] == -1 and g["a"][7] == -1
    assert sum(int(x) >= 0 for x in g["a"]) == tin.B - 2


def test_tree_per_request_temperatures_alone():
    # temperatures alone: no select, the walk takes each request's own statistics; equal
    # values give the scalar call's results bit for bit
    tin = synth.make_tree(seed=136, B=10, V=50000, dtype="bf16", n_range=(2, 18))
    temps = np.array([0.4, 0.7, 1.0, 1.5, 0.7, 2.0, 0.9, 0.7, 1.1, 0.6], np.float32)
    _check(tin, temps=temps)
    same = TreeOnDevice(tin, temps=np.full(tin.B, tin.T, np.float32)).run()
    ref = TreeOnDevice(tin).run()
    for key in ("a", "n", "out", "nodes", "flags"):
        assert np.array_equal(same[key], ref[key]), key


def _cycle(tin, seed):
    """Append (pending token + every node), verify the tree, commit the accepted paths."""
    rec = synth.KVRecipe(L=2, H=2, D=8, prefix_lo=20, prefix_hi=120, share_group=2,
                         share_blocks=1)
    kv = synth.make_kv("c1", tin, seed=seed, recipe=rec)
    d = dev()
    pool = pool_tensor(kv, d)
    cache = binding.PagedKVCache(pool, _t(kv.block_tables.astype(np.int32), d),
                                 _t(kv.seq_lens.astype(np.int32), d),
                                 _t(kv.refcount.astype(np.int32), d),
                                 _t(kv.free_list.astype(np.int32), d),
                                 torch.tensor([kv.free_count], dtype=torch.int32, device=d),
                                 torch.zeros(1, dtype=torch.int32, device=d))
    k_new = torch.from_numpy(kv.k_new.view(np.int16)).view(torch.bfloat16).to(d)
    v_new = torch.from_numpy(kv.v_new.view(np.int16)).view(torch.bfloat16).to(d)
    ws = torch.empty(binding.kv_paged_append_workspace_size(tin.B, k_new.shape[1]),
                     dtype=torch.uint8, device=d)
    binding.kv_paged_append(cache, k_new, v_new, _t(kv.cu_new, d), ws)
    t = TreeOnDevice(tin)
    g = t.run()
    binding.kv_tree_commit(cache, t.num_acc, t.nodes, t.cu)
    torch.cuda.synchronize()
    meta = dict(tables=cache.block_tables.cpu().numpy(), seq_lens=cache.seq_lens.cpu().numpy(),
                refcount=cache.refcount.cpu().numpy(), free_list=cache.free_list.cpu().numpy(),
                free_count=int(cache.free_count.item()), state=int(cache.state.item()))
    o_kv = oracle.PagedKV(kv.L, kv.H, kv.D, kv.block_size, kv.num_blocks, kv.block_tables,
                          kv.seq_lens, kv.refcount, kv.free_list, kv.free_count, kv.blocks)
    assert o_kv.append(kv.k_new, kv.v_new, kv.cu_new) == 0
    return kv, g, meta, pool, o_kv


@pytest.mark.parametrize("seed", [0, 1])
def test_tree_cycle_keeps_the_accepted_path(seed):
    tin = synth.make_tree(seed=120 + seed, B=10, V=8000, n_range=(0, 12), noise_std=0.5)
    kv, g, meta, pool, o_kv = _cycle(tin, seed)
    o = oracle.tree_verify_batch(tin.target, tin.draft, tin.tokens, tin.parent, tin.cu_nodes,
                                 tin.u_accept, tin.u_sample, tin.T, tin.max_nodes, tin.dtype)
    errs, fl, mism = compare_tree(tin, g, o)
    assert not errs, "\n".join(errs[:20])
    # the oracle's cache takes the GPU's paths
    assert oracle.tree_commit(o_kv, g["a"], g["nodes"][:tin.N], tin.cu_nodes) == 0
    errs = compare_kv_meta(o_kv, meta, f"tree seed {seed}") + compare_kv_data(o_kv, pool, kv)
    assert not errs, "\n".join(errs[:20])
    o_kv.check_invariants()
    # and the kept entries are the pending token's and the path's, in path order
    for b in range(tin.B):
        lo, a = int(tin.cu_nodes[b]), int(g["a"][b])
        s0 = int(kv.seq_lens[b])
        view = o_kv.logical_view(b, s0)
        rows = [lo + b] + [lo + b + 1 + int(j) for j in g["nodes"][lo: lo + a]]
        want = np.stack([kv.k_new[:, rows], kv.v_new[:, rows]], axis=1)
        assert np.array_equal(view, want)


def test_tree_commit_rejects_unsound_paths():
    tin = synth.make_tree(seed=122, B=4, V=2000, dtype="f32", n_range=(3, 6))
    kv, g, meta, pool, o_kv = _cycle(tin, 3)
    # a second commit with a path that is not increasing, on a fresh copy of the state
    d = dev()
    cache = binding.PagedKVCache(pool, _t(meta["tables"], d), _t(meta["seq_lens"], d),
                                 _t(meta["refcount"], d), _t(meta["free_list"], d),
                                 torch.tensor([meta["free_count"]], dtype=torch.int32, device=d),
                                 torch.zeros(1, dtype=torch.int32, device=d))
    nodes = torch.zeros(tin.N, dtype=torch.int32, device=d)      # all zeros: not increasing
    num = torch.full((tin.B,), 2, dtype=torch.int32, device=d)
    binding.kv_tree_commit(cache, num, nodes, _t(tin.cu_nodes, d))
    torch.cuda.synchronize()
    assert np.array_equal(cache.seq_lens.cpu().numpy(), meta["seq_lens"])
    assert int(cache.state.item()) & binding.KV_ERR_ROLLBACK


@pytest.mark.parametrize("dtype,V", [("bf16", 128256), ("f32", 32000), ("bf16", 4001)])
def test_team_sizes_give_identical_results(dtype, V):
    # every member combines the chunk partials in one fixed order, so the walk, the draw
    # and the flags do not depend on how many workgroups share a request (more members
    # than chunks included) or on what the workspace held before the call
    tin = synth.make_tree(seed=113, B=6, V=V, dtype=dtype, n_range=(5, 30))
    log(f"[tree-team] B={tin.B} N={tin.N} V={V} {dtype}: team 1")
    ref = TreeOnDevice(tin, team=1).run()
    o = oracle.tree_verify_batch(tin.target, tin.draft, tin.tokens, tin.parent, tin.cu_nodes,
                                 tin.u_accept, tin.u_sample, tin.T, tin.max_nodes, tin.dtype)
    errs, _, _ = compare_tree(tin, ref, o)
    assert not errs, "\n".join(errs[:20])
    for team in (2, 3, 5, 8, 16, 0):
        log(f"[tree-team]   team {team}")
        g = TreeOnDevice(tin, team=team, ws_fill=0xAB).run()
        for key in ("a", "n", "out", "nodes", "flags"):
            assert np.array_equal(g[key], ref[key]), (team, key)
        assert g["err"] == ref["err"], team


def test_team_wait_bound_fails_requests_cleanly(monkeypatch):
    # the team's wait is bounded: with a bound of zero polls, members that would wait for
    # the others give up, and their requests fail with SPECDEC_ERR_TEAM (num_accepted -1,
    # nothing emitted) while every other request keeps the normal result; the launch ends
    tin = synth.make_tree(seed=114, B=8, V=128256, dtype="bf16", n_range=(10, 30))
    ref = TreeOnDevice(tin, team=4).run()
    monkeypatch.setenv("SPECDEC_TREE_SPIN_LIMIT", "0")
    log("[tree-team] wait bound 0 polls, team 4")
    g = TreeOnDevice(tin, team=4).run()
    monkeypatch.delenv("SPECDEC_TREE_SPIN_LIMIT")
    failed = [b for b in range(tin.B) if g["flags"][b] & binding.ERR_TEAM]
    log(f"[tree-team]   {len(failed)} of {tin.B} requests gave up")
    assert failed, "a zero-poll bound should make some member give up"
    for b in range(tin.B):
        if b in failed:
            assert g["a"][b] == -1 and g["n"][b] == 0
        else:
            assert g["a"][b] == ref["a"][b] and g["n"][b] == ref["n"][b]
            lo = int(tin.cu_nodes[b])
            n = int(ref["n"][b])
            assert np.array_equal(g["out"][lo + b: lo + b + n], ref["out"][lo + b: lo + b + n])
            assert np.array_equal(g["nodes"][lo: lo + n - 1], ref["nodes"][lo: lo + n - 1])
            assert g["flags"][b] == ref["flags"][b]
    assert g["err"] & binding.ERR_TEAM
    # and a normal call afterwards is unaffected
    again = TreeOnDevice(tin, team=4).run()
    for key in ("a", "n", "out", "nodes", "flags"):
        assert np.array_equal(again[key], ref[key]), key
