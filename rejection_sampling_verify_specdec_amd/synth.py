"""Seeded synthetic inputs for the verification step and the paged KV cache.

This module only draws random data and lays it out; it holds none of the verification
arithmetic (no softmax, accept test or inverse CDF) and imports neither the HIP binding
nor the oracle, so both sides of a parity test can be fed from it.

Draft tokens stand in for the draft model's proposals: y_i is drawn from the draft
distribution q_i after the same temperature / top-k transform, using the Gumbel-max
method (argmax of z/T plus independent Gumbel noise over the kept tokens), which samples
that distribution exactly without normalizing it.

Workload recipes (the pages publish no benchmark or dataset; these synthetic shapes stand
in for real target / draft logits and K/V):

=====  ============================================================================
tiny   B=1, k=4, V=1000 fp32, target N(0,2) at 5 rows, draft = target + N(0,1), T=1
c1     B=64, k=5, V=32000 fp32, as tiny; KV 1 layer x 8 heads x 128, prefix U[100,2000]
c2     B=256, k=5, V=128256 bf16, target N(0,3), draft = target + N(0,1.5), T=0.7;
       KV 32 layers x 8 x 128 bf16, block 16, prefix U[512,4096]
c3     B=512, k_b ~ U{1..8}, V=152064 bf16, T=1; 20% draft = bitwise target copy,
       20% draft noise N(0,4), 60% N(0,1.5); target N(0,3); KV as c2; prefixes of
       rejected requests placed so the discarded range starts a fresh 16-slot block
c4     B=128, k=8, V=128256 bf16, T=0.8, top-k 64; target N(0,3), draft noise N(0,1);
       KV as c2 with prefix U[1024,8192]; groups of 4 requests share their first 32 full
       blocks (refcount 4)
=====  ============================================================================

"N(0,s)" is read as standard deviation s. Random draws come from
``numpy.random.default_rng(seed)`` in a fixed order (k_b, request classes, target
logits, draft noise, Gumbel uniforms, u_accept, u_sample) and the KV state from
``default_rng([seed, 7])`` (prefix lengths, block permutation, prefix contents, new K/V).
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class KVRecipe:
    L: int = 32
    H: int = 8
    D: int = 128
    block_size: int = 16
    prefix_lo: int = 512
    prefix_hi: int = 4096
    share_group: int = 0          # requests per shared-prefix group (0 = no sharing)
    share_blocks: int = 0         # leading full blocks shared inside a group
    align_rejections: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    V: int
    dtype: str                    # "f32" or "bf16"
    T: float
    top_k: int = 0
    k: int = 0                    # uniform proposals per request
    k_range: Optional[Tuple[int, int]] = None   # ragged k_b ~ U{lo..hi}
    target_std: float = 3.0
    # draft classes: (fraction, kind, noise std); kind "noise" = target + N(0, std),
    # "copy" = bitwise copy of the target rows
    classes: Tuple[Tuple[float, str, float], ...] = ((1.0, "noise", 1.0),)
    kv: Optional[KVRecipe] = None

    @property
    def max_k(self) -> int:
        return self.k_range[1] if self.k_range else self.k


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", B=1, V=1000, dtype="f32", T=1.0, k=4, target_std=2.0,
                     classes=((1.0, "noise", 1.0),)),
    "c1": Workload("c1", B=64, V=32000, dtype="f32", T=1.0, k=5, target_std=2.0,
                   classes=((1.0, "noise", 1.0),),
                   kv=KVRecipe(L=1, prefix_lo=100, prefix_hi=2000)),
    "c2": Workload("c2", B=256, V=128256, dtype="bf16", T=0.7, k=5, target_std=3.0,
                   classes=((1.0, "noise", 1.5),), kv=KVRecipe()),
    "c3": Workload("c3", B=512, V=152064, dtype="bf16", T=1.0, k_range=(1, 8),
                   target_std=3.0,
                   classes=((0.2, "copy", 0.0), (0.2, "noise", 4.0), (0.6, "noise", 1.5)),
                   kv=KVRecipe(align_rejections=True)),
    "c4": Workload("c4", B=128, V=128256, dtype="bf16", T=0.8, top_k=64, k=8,
                   target_std=3.0, classes=((1.0, "noise", 1.0),),
                   kv=KVRecipe(prefix_lo=1024, prefix_hi=8192, share_group=4,
                               share_blocks=32)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); bit patterns as uint16."""
    x = np.asarray(x, dtype=np.float32)
    u = np.ascontiguousarray(x).reshape(-1).view(np.uint32)
    r = np.empty(u.shape, dtype=np.uint16)
    # in 32 bits: every non-NaN pattern is <= 0xFF800000, so adding <= 0x8000 cannot wrap
    # (NaN lanes are replaced below); chunked to bound the temporaries
    step = 1 << 22
    for s in range(0, u.size, step):
        t = u[s:s + step] >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += u[s:s + step]
        t >>= np.uint32(16)
        r[s:s + step] = t
    r = r.reshape(x.shape)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class VerifyInputs:
    wl: Workload
    B: int
    V: int
    K: int
    max_k: int
    dtype: str
    T: float
    top_k: int
    target: np.ndarray            # [K+B, V] float32, or uint16 bf16 bits
    draft: np.ndarray             # [K, V]
    draft_tokens: np.ndarray      # int32 [K]
    cu_draft: np.ndarray          # int32 [B+1]
    u_accept: np.ndarray          # float32 [K]
    u_sample: np.ndarray          # float32 [B]
    kinds: List[str] = field(default_factory=list)

    @property
    def k_b(self) -> np.ndarray:
        return np.diff(self.cu_draft)

    def rows_as_f32(self, which: str, rows: slice) -> np.ndarray:
        x = self.target[rows] if which == "target" else self.draft[rows]
        return bf16_bits_to_f32(x) if self.dtype == "bf16" else x


def _gumbel_sample(z: np.ndarray, T: float, top_k: int, rng: np.random.Generator) -> np.ndarray:
    """Draft proposals: one token per row of z ([R, V] float32) from softmax(z/T) over the
    top-k kept set (ties inclusive), by Gumbel-max."""
    R, V = z.shape
    out = np.empty(R, dtype=np.int32)
    step = 128
    for r0 in range(0, R, step):
        zz = z[r0:r0 + step].astype(np.float64) / T
        if 0 < top_k < V:
            thr = np.partition(zz, V - top_k, axis=1)[:, V - top_k][:, None]
            zz = np.where(zz >= thr, zz, -np.inf)
        u = rng.random(zz.shape)
        with np.errstate(divide="ignore"):
            g = -np.log(-np.log(u))
        out[r0:r0 + step] = np.argmax(zz + g, axis=1)
    return out


def make_verify(wl, seed: int = 0, B: Optional[int] = None, V: Optional[int] = None,
                **over) -> VerifyInputs:
    """Draw one verification batch for workload ``wl`` (a name or a Workload).

    ``B`` / ``V`` shrink the batch or vocabulary for quick tests; other fields of the
    workload can be overridden by keyword (e.g. ``T=0.5``, ``top_k=8``)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if B is not None or V is not None or over:
        wl = replace(wl, B=B if B is not None else wl.B, V=V if V is not None else wl.V, **over)
    rng = np.random.default_rng(seed)
    B, Vv = wl.B, wl.V
    if wl.k_range:
        k_b = rng.integers(wl.k_range[0], wl.k_range[1] + 1, size=B)
    else:
        k_b = np.full(B, wl.k, dtype=np.int64)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(k_b)
    K = int(cu[-1])
    # request classes by a seeded permutation
    perm = rng.permutation(B)
    kinds: List[str] = [""] * B
    noise_std = np.zeros(B, dtype=np.float32)
    start = 0
    for i, (frac, kind, std) in enumerate(wl.classes):
        cnt = B - start if i == len(wl.classes) - 1 else int(round(frac * B))
        for b in perm[start:start + cnt]:
            kinds[b] = kind
            noise_std[b] = std
        start += cnt
    target32 = rng.standard_normal((K + B, Vv), dtype=np.float32)
    target32 *= np.float32(wl.target_std)
    req_of_draft = np.repeat(np.arange(B), k_b)
    t_of_d = np.arange(K) + req_of_draft
    draft32 = rng.standard_normal((K, Vv), dtype=np.float32)
    draft32 *= noise_std[req_of_draft][:, None]
    draft32 += target32[t_of_d]
    if wl.dtype == "bf16":
        target = f32_to_bf16_bits(target32)
        draft = f32_to_bf16_bits(draft32)
        copy_rows = np.array([kinds[b] == "copy" for b in req_of_draft], dtype=bool)
        if copy_rows.any():
            draft[copy_rows] = target[t_of_d[copy_rows]]
        draft_vals = bf16_bits_to_f32(draft)
    else:
        target, draft = target32, draft32
        copy_rows = np.array([kinds[b] == "copy" for b in req_of_draft], dtype=bool)
        if copy_rows.any():
            draft[copy_rows] = target[t_of_d[copy_rows]]
        draft_vals = draft
    del target32, draft32
    tokens = _gumbel_sample(draft_vals, float(np.float32(wl.T)), wl.top_k, rng) if K else \
        np.zeros(0, dtype=np.int32)
    u_accept = rng.random(K, dtype=np.float32)
    u_sample = rng.random(B, dtype=np.float32)
    return VerifyInputs(wl, B, Vv, K, wl.max_k, wl.dtype, float(np.float32(wl.T)), wl.top_k,
                        np.ascontiguousarray(target), np.ascontiguousarray(draft),
                        tokens.astype(np.int32), cu, u_accept, u_sample, kinds)


@dataclass
class KVInputs:
    L: int
    H: int
    D: int
    block_size: int
    num_blocks: int
    max_blocks_per_req: int
    block_tables: np.ndarray      # int32 [B][MBR], -1 = none
    seq_lens: np.ndarray          # int32 [B]
    refcount: np.ndarray          # int32 [NB]
    free_list: np.ndarray         # int32 [NB]; entries [0, free_count) are the stack
    free_count: int
    k_new: np.ndarray             # uint16 bf16 bits [L][N][H][D]
    v_new: np.ndarray
    cu_new: np.ndarray            # int32 [B+1]; n_b = k_b + 1
    blocks: Dict[int, Tuple[np.ndarray, np.ndarray]]   # bid -> (uint16 [L][2][bs][H][D], defined[bs])


def make_kv(wl, vin: VerifyInputs, seed: int = 0, a_hint: Optional[np.ndarray] = None,
            cycles: int = 1, recipe: Optional[KVRecipe] = None) -> KVInputs:
    """Paged-cache state before one cycle, and the candidate K/V the target pass produced.

    ``a_hint`` (accepted counts) places each rejected request's prefix so that its
    discarded range starts at a 16-slot block boundary when the recipe asks for it.
    ``cycles`` sizes the free pool and block tables for that many back-to-back cycles."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    kv = recipe or wl.kv
    rng = np.random.default_rng([seed, 7])
    B, bs = vin.B, kv.block_size
    k_b = vin.k_b.astype(np.int64)
    pre = rng.integers(kv.prefix_lo, kv.prefix_hi + 1, size=B).astype(np.int64)
    if a_hint is not None and kv.align_rejections:
        for b in range(B):
            a = int(a_hint[b])
            if 0 <= a < k_b[b]:
                p = pre[b] - ((pre[b] + 1 + a) % bs)
                if p < kv.prefix_lo:
                    p += bs
                pre[b] = p
    if kv.share_group > 1:
        # keep every request of a group past the shared region
        pre = np.maximum(pre, kv.share_blocks * bs + 1)
    nblk = -(-pre // bs)
    grow = cycles * (k_b + 1)
    MBR = int(-(-(pre + grow).max() // bs)) + 1
    shared_of: Dict[int, int] = {}
    distinct = 0
    for b in range(B):
        for lb in range(int(nblk[b])):
            if kv.share_group > 1 and lb < kv.share_blocks and b % kv.share_group != 0:
                continue
            distinct += 1
    headroom = int(np.sum(-(-(pre + grow) // bs) - nblk + 1))
    NB = distinct + headroom
    perm = rng.permutation(NB).astype(np.int32)
    tables = np.full((B, MBR), -1, dtype=np.int32)
    refcount = np.zeros(NB, dtype=np.int32)
    nxt = 0
    for b in range(B):
        for lb in range(int(nblk[b])):
            if kv.share_group > 1 and lb < kv.share_blocks and b % kv.share_group != 0:
                X = int(tables[b - b % kv.share_group, lb])
            else:
                X = int(perm[nxt])
                nxt += 1
            tables[b, lb] = X
            refcount[X] += 1
    free_list = np.zeros(NB, dtype=np.int32)
    free_count = NB - nxt
    free_list[:free_count] = perm[nxt:]
    L, H, D = kv.L, kv.H, kv.D
    blocks: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
    for b in range(B):
        off = int(pre[b] % bs)
        if off:
            X = int(tables[b, pre[b] // bs])
            if X in blocks:
                continue
            data = np.zeros((L, 2, bs, H, D), dtype=np.uint16)
            data[:, :, :off] = f32_to_bf16_bits(
                rng.standard_normal((L, 2, off, H, D), dtype=np.float32))
            defined = np.zeros(bs, dtype=bool)
            defined[:off] = True
            blocks[X] = (data, defined)
    N = vin.K + B
    k_new = f32_to_bf16_bits(rng.standard_normal((L, N, H, D), dtype=np.float32))
    v_new = f32_to_bf16_bits(rng.standard_normal((L, N, H, D), dtype=np.float32))
    cu_new = (vin.cu_draft.astype(np.int64) + np.arange(B + 1)).astype(np.int32)
    return KVInputs(L, H, D, bs, NB, MBR, tables, pre.astype(np.int32), refcount, free_list,
                    int(free_count), k_new, v_new, cu_new, blocks)


@dataclass
class TreeInputs:
    """A batch of draft trees: request b owns nodes cu_nodes[b] .. cu_nodes[b+1]-1 and the
    target / draft rows cu_nodes[b] + b + v of its positions v = 0 (root) .. n_b."""
    B: int
    V: int
    N: int
    max_nodes: int
    dtype: str
    T: float
    target: np.ndarray            # [N+B, V] float32, or uint16 bf16 bits
    draft: np.ndarray             # [N+B, V]
    tokens: np.ndarray            # int32 [N]
    parent: np.ndarray            # int32 [N], -1 or an earlier node of the request
    cu_nodes: np.ndarray          # int32 [B+1]
    u_accept: np.ndarray          # float32 [N]
    u_sample: np.ndarray          # float32 [B]

    # the names the cache generator reads: one cache entry per node plus the pending token
    @property
    def K(self) -> int:
        return self.N

    @property
    def cu_draft(self) -> np.ndarray:
        return self.cu_nodes

    @property
    def k_b(self) -> np.ndarray:
        return np.diff(self.cu_nodes)


def make_tree(seed: int = 0, B: int = 16, V: int = 32000, dtype: str = "bf16", T: float = 0.7,
              n_range=(1, 16), target_std: float = 3.0, noise_std: float = 1.5,
              branch: float = 0.5, max_nodes: int = 64, top_k: int = 0) -> TreeInputs:
    """Seeded trees: node j's parent is j - 1 (the chain goes on) or, with probability
    ``branch``, a uniform pick among the root and the earlier nodes. Target rows N(0,
    target_std) per position, draft rows the target row plus N(0, noise_std); each node's
    token is a Gumbel-max draw from the draft row of its parent's position (siblings are
    independent draws; within the row's top_k when given), standing in for the draft
    model."""
    rng = np.random.default_rng(seed)
    n_b = rng.integers(n_range[0], n_range[1] + 1, size=B)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(n_b)
    N = int(cu[-1])
    parent = np.zeros(N, dtype=np.int32)
    for b in range(B):
        for j in range(int(n_b[b])):
            if j == 0:
                parent[cu[b]] = -1
            elif rng.random() < branch:
                parent[cu[b] + j] = int(rng.integers(-1, j))
            else:
                parent[cu[b] + j] = j - 1
    target32 = rng.standard_normal((N + B, V), dtype=np.float32) * np.float32(target_std)
    draft32 = target32 + rng.standard_normal((N + B, V), dtype=np.float32) * np.float32(noise_std)
    if dtype == "bf16":
        target, draft = f32_to_bf16_bits(target32), f32_to_bf16_bits(draft32)
        dvals = bf16_bits_to_f32(draft)
    else:
        target, draft, dvals = target32, draft32, draft32
    # the draft row each node was drawn from: its parent's position
    req = np.repeat(np.arange(B), n_b)
    rows = cu[req] + req + parent + 1
    tokens = _gumbel_sample(dvals[rows], float(np.float32(T)), top_k, rng) if N else \
        np.zeros(0, dtype=np.int32)
    u_accept = rng.random(N, dtype=np.float32)
    u_sample = rng.random(B, dtype=np.float32)
    return TreeInputs(B, V, N, max_nodes, dtype, float(np.float32(T)), np.ascontiguousarray(target),
                      np.ascontiguousarray(draft), tokens.astype(np.int32), parent, cu, u_accept,
                      u_sample)


# Tree workloads: B requests with U{n_lo..n_hi}-node trees (children of a node are
# independent draws from its draft row), target N(0, target_std), draft = target +
# N(0, noise_std), bf16 rows; paged KV as the headline workload.
TREE_WORKLOADS = {
    "t1": dict(B=128, V=128256, dtype="bf16", T=0.7, n_range=(8, 24), target_std=3.0,
               noise_std=0.5, branch=0.5),
    # a small serving batch: latency of one step rather than throughput
    "t2": dict(B=8, V=128256, dtype="bf16", T=0.7, n_range=(8, 24), target_std=3.0,
               noise_std=0.5, branch=0.5),
}
