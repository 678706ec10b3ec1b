"""Thin ctypes binding of ``libspecdec.so`` (see ``include/specdec.h``).

Argument marshalling only: torch tensors are checked for device, dtype, shape and
contiguity, and their device pointers plus torch's current HIP stream are passed to the C
entry points of the same names. Every step of the path runs in the library's kernels.
The library must have been built (``python -m rejection_sampling_verify_specdec_amd.build``);
calls fail loudly otherwise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecdec.so")

SPECDEC_OK = 0
SPECDEC_EINVAL = -1
SPECDEC_EHIP = -3
SPECDEC_EWORKSPACE = -4
SPECDEC_ESCRATCH = -5
STATIC_SCRATCH_BYTES = 8 << 20
SPECDEC_F32 = 0
SPECDEC_BF16 = 1

ERR_TOKEN = 1
ERR_K = 2
ERR_NONFINITE = 4
ERR_QZERO = 8
ERR_ZFALLBACK = 16
ERR_UNIFORM = 32
ERR_PARAM = 64
ERR_TREE = 128
ERR_TEAM = 256
MAX_TREE = 64
MAX_TREE_TEAM = 16
KV_ERR_NOMEM = 64
KV_ERR_APPEND = 128
KV_ERR_ROLLBACK = 256
KV_APPEND_REJECTED = 1 << 16

MAX_K = 64
# positions the early-exit calls read one launch at a time before one launch reads the rest
# of every request still live (SPECDEC_EARLY_EXIT_SEQUENTIAL)
EARLY_EXIT_SEQUENTIAL = 2
MAX_KV_BATCH = 4096
MAX_V = 2097152

EXPORTED = [
    "specdec_status_string", "specdec_verify_workspace_size", "specdec_verify",
    "specdec_verify_early_exit",
    "kv_paged_append_workspace_size", "kv_paged_append", "kv_rollback", "kv_rollback_draft",
    "specdec_cycle_workspace_size", "specdec_cycle", "specdec_cycle_early_exit",
    "specdec_cycle_static",
    "specdec_tree_verify_workspace_size",
    "specdec_tree_verify", "kv_tree_commit",
    "kv_contig_append", "kv_contig_rollback",
    "specdec_probe_read", "specdec_probe_copy",
]


class SpecdecError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


class SpecdecDebug(ctypes.Structure):
    _fields_ = [
        ("p_y", ctypes.c_void_p), ("q_y", ctypes.c_void_p),
        ("row_max", ctypes.c_void_p), ("row_sum", ctypes.c_void_p),
        ("row_thr", ctypes.c_void_p), ("row_nkept", ctypes.c_void_p),
        ("resid_mass", ctypes.c_void_p), ("picked_prob", ctypes.c_void_p),
        ("req_flags", ctypes.c_void_p),
        ("ev_stats_begin", ctypes.c_void_p), ("ev_stats_end", ctypes.c_void_p),
        ("ev_stats_done", ctypes.c_void_p),
        ("accept_prob", ctypes.c_void_p), ("expected_emitted", ctypes.c_void_p),
    ]


class SpecdecParams(ctypes.Structure):
    """Per-request transform arrays (device pointers, or None for the scalar)."""
    _fields_ = [
        ("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
        ("top_k_max", ctypes.c_int32),
        ("eos_token", ctypes.c_void_p), ("max_emit", ctypes.c_void_p),
    ]


def _params(B: int, dev, temperatures, top_ks, top_ps, top_k_max, eos_tokens=None,
            max_emit=None):
    """SpecdecParams for optional per-request tensors, or None when none is given."""
    if all(x is None for x in (temperatures, top_ks, top_ps, eos_tokens, max_emit)):
        return None
    if eos_tokens is not None:
        _check(eos_tokens, "eos_tokens", torch.int32, B, dev)
    if max_emit is not None:
        _check(max_emit, "max_emit", torch.int32, B, dev)
    if temperatures is not None:
        _check(temperatures, "temperatures", torch.float32, B, dev)
    if top_ks is not None:
        _check(top_ks, "top_ks", torch.int32, B, dev)
        if top_k_max is None:
            raise ValueError("top_k_max is required with top_ks")
    if top_ps is not None:
        _check(top_ps, "top_ps", torch.float32, B, dev)
    opt = lambda t: _ptr(t) if t is not None else None
    return SpecdecParams(opt(temperatures), opt(top_ks), opt(top_ps),
                         int(top_k_max) if top_k_max is not None else 0, opt(eos_tokens),
                         opt(max_emit))


class KvPagedCacheStruct(ctypes.Structure):
    _fields_ = [
        ("pool", ctypes.c_void_p),
        ("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("max_blocks_per_req", ctypes.c_int32),
        ("block_tables", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("refcount", ctypes.c_void_p), ("free_list", ctypes.c_void_p),
        ("free_count", ctypes.c_void_p), ("state", ctypes.c_void_p),
    ]


class KvContigCacheStruct(ctypes.Structure):
    _fields_ = [
        ("pool", ctypes.c_void_p),
        ("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_len", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p), ("state", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library once; raise if it was not built. The path defaults to the in-tree
    build; SPECDEC_LIBRARY names another build of the same sources (the host-sanitized one
    the CPU tests load)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("SPECDEC_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m rejection_sampling_verify_specdec_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.specdec_status_string.argtypes = [ctypes.c_int]
    lib.specdec_status_string.restype = ctypes.c_char_p
    f32 = ctypes.c_float
    pp = ctypes.POINTER(SpecdecParams)
    lib.specdec_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32, f32, pp]
    lib.specdec_verify_workspace_size.restype = sz
    for fn in (lib.specdec_verify, lib.specdec_verify_early_exit):
        fn.argtypes = [vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, f32, pp, vp,
                       vp, vp, vp, ctypes.POINTER(SpecdecDebug), vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.kv_paged_append_workspace_size.argtypes = [i32, i32]
    lib.kv_paged_append_workspace_size.restype = sz
    lib.kv_paged_append.argtypes = [ctypes.POINTER(KvPagedCacheStruct), i32, vp, vp, vp, i32,
                                    vp, sz, vp]
    lib.kv_paged_append.restype = ctypes.c_int
    for fn in (lib.kv_rollback, lib.kv_rollback_draft):
        fn.argtypes = [ctypes.POINTER(KvPagedCacheStruct), i32, vp, vp, vp]
        fn.restype = ctypes.c_int
    lib.specdec_cycle_workspace_size.argtypes = [i32, i32, i32, i32, i32, f32, pp]
    lib.specdec_cycle_workspace_size.restype = sz
    for fn in (lib.specdec_cycle, lib.specdec_cycle_early_exit):
        fn.argtypes = [ctypes.POINTER(KvPagedCacheStruct), vp, vp, vp, vp, i32, vp, vp, vp, vp,
                       i32, i32, i32, i32, f32, i32, f32, pp, vp, vp, vp, vp,
                       ctypes.POINTER(SpecdecDebug), vp, sz, vp]
        fn.restype = ctypes.c_int
    lib.specdec_cycle_static.argtypes = [ctypes.POINTER(KvPagedCacheStruct), vp, vp, vp, vp, i32,
                                         vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, f32, pp,
                                         vp, vp, vp, vp, ctypes.POINTER(SpecdecDebug), vp]
    lib.specdec_cycle_static.restype = ctypes.c_int
    lib.specdec_tree_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32, f32, pp]
    lib.specdec_tree_verify_workspace_size.restype = sz
    lib.specdec_tree_verify.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                        i32, f32, pp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.specdec_tree_verify.restype = ctypes.c_int
    lib.kv_tree_commit.argtypes = [ctypes.POINTER(KvPagedCacheStruct), i32, vp, vp, vp, i32, vp]
    lib.kv_tree_commit.restype = ctypes.c_int
    lib.kv_contig_append.argtypes = [ctypes.POINTER(KvContigCacheStruct), i32, vp, vp, vp, i32, vp]
    lib.kv_contig_append.restype = ctypes.c_int
    lib.kv_contig_rollback.argtypes = [ctypes.POINTER(KvContigCacheStruct), i32, vp, vp, i32, vp]
    lib.kv_contig_rollback.restype = ctypes.c_int
    lib.specdec_probe_read.argtypes = [vp, sz, vp, vp]
    lib.specdec_probe_read.restype = ctypes.c_int
    lib.specdec_probe_copy.argtypes = [vp, vp, sz, vp]
    lib.specdec_probe_copy.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().specdec_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, numel: Optional[int] = None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, is on {t.device}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")


def _logits_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPECDEC_BF16
    if t.dtype == torch.float32:
        return SPECDEC_F32
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _pref(params):
    return ctypes.byref(params) if params is not None else None


def specdec_verify_workspace_size(B: int, K: int, V: int, dtype: int, top_k: int,
                                  top_p: float = 1.0, params: Optional[SpecdecParams] = None) -> int:
    return int(load_library().specdec_verify_workspace_size(B, K, V, dtype, top_k, float(top_p),
                                                            _pref(params)))


def specdec_verify(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                   draft_tokens: torch.Tensor, cu_draft: torch.Tensor,
                   u_accept: torch.Tensor, u_sample: torch.Tensor, *, max_k: int,
                   temperature: float, top_k: int, out_tokens: torch.Tensor,
                   num_accepted: torch.Tensor, num_emitted: torch.Tensor,
                   err_word: torch.Tensor, workspace: torch.Tensor,
                   debug: Optional[SpecdecDebug] = None, top_p: float = 1.0,
                   temperatures: Optional[torch.Tensor] = None,
                   top_ks: Optional[torch.Tensor] = None, top_ps: Optional[torch.Tensor] = None,
                   top_k_max: Optional[int] = None, eos_tokens: Optional[torch.Tensor] = None,
                   max_emit: Optional[torch.Tensor] = None, early_exit: bool = False) -> None:
    """Enqueue one verification step on torch's current stream (shapes as in the header).
    temperatures / top_ks / top_ps: optional per-request [B] device tensors replacing the
    scalars (top_k_max bounds the active top_ks). ``early_exit``
    (specdec_verify_early_exit): no row is read past a request's first rejection."""
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be a GPU tensor")
    dtype = _logits_dtype(target_logits)
    if target_logits.dim() != 2:
        raise ValueError("target_logits must be [K+B, V]")
    B = cu_draft.numel() - 1
    R, V = target_logits.shape
    K = R - B
    _check(target_logits, "target_logits", target_logits.dtype, device=dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, K * V, dev)
    _check(draft_tokens, "draft_tokens", torch.int32, K, dev)
    _check(cu_draft, "cu_draft", torch.int32, B + 1, dev)
    _check(u_accept, "u_accept", torch.float32, K, dev)
    _check(u_sample, "u_sample", torch.float32, B, dev)
    _check(out_tokens, "out_tokens", torch.int32, K + B, dev)
    _check(num_accepted, "num_accepted", torch.int32, B, dev)
    _check(num_emitted, "num_emitted", torch.int32, B, dev)
    _check(err_word, "err_word", torch.int32, 1, dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    prm = _params(B, dev, temperatures, top_ks, top_ps, top_k_max, eos_tokens, max_emit)
    name = "specdec_verify_early_exit" if early_exit else "specdec_verify"
    st = getattr(lib, name)(
        _ptr(target_logits), _ptr(draft_logits), dtype, _ptr(draft_tokens), _ptr(cu_draft),
        _ptr(u_accept), _ptr(u_sample), B, K, max_k, V, float(temperature), int(top_k),
        float(top_p), _pref(prm), _ptr(out_tokens), _ptr(num_accepted), _ptr(num_emitted), _ptr(err_word),
        ctypes.byref(debug) if debug is not None else None,
        _ptr(workspace), workspace.numel(), _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError(name, st)


class PagedKVCache:
    """Device tensors of one paged cache plus the C struct that points at them."""

    def __init__(self, pool: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                 refcount: torch.Tensor, free_list: torch.Tensor, free_count: torch.Tensor,
                 state: torch.Tensor):
        if pool.dtype != torch.bfloat16 or pool.dim() != 6:
            raise ValueError("pool must be bf16 [L][2][NB][block_size][H][D]")
        L, two, NB, bs, H, D = pool.shape
        if two != 2:
            raise ValueError("pool dim 1 must be 2 (K, V)")
        dev = pool.device
        _check(pool, "pool", torch.bfloat16, device=dev)
        _check(block_tables, "block_tables", torch.int32, device=dev)
        _check(seq_lens, "seq_lens", torch.int32, device=dev)
        _check(refcount, "refcount", torch.int32, NB, dev)
        _check(free_list, "free_list", torch.int32, NB, dev)
        _check(free_count, "free_count", torch.int32, 1, dev)
        _check(state, "state", torch.int32, 1, dev)
        self.pool, self.block_tables, self.seq_lens = pool, block_tables, seq_lens
        self.refcount, self.free_list, self.free_count, self.state = refcount, free_list, free_count, state
        self.device = dev
        self.struct = KvPagedCacheStruct(
            pool.data_ptr(), L, H, D, bs, NB, block_tables.shape[1],
            block_tables.data_ptr(), seq_lens.data_ptr(), refcount.data_ptr(),
            free_list.data_ptr(), free_count.data_ptr(), state.data_ptr())


def kv_paged_append_workspace_size(B: int, N: int) -> int:
    return int(load_library().kv_paged_append_workspace_size(B, N))


def kv_paged_append(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                    cu_new: torch.Tensor, workspace: torch.Tensor) -> None:
    """Enqueue the provisional append of k_new / v_new ([L][N][H][D] bf16)."""
    lib = load_library()
    dev = cache.device
    B = cu_new.numel() - 1
    N = k_new.shape[1]
    s = cache.struct
    shape = (s.num_layers, N, s.num_kv_heads, s.head_dim)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new / v_new must be {shape}")
    _check(k_new, "k_new", torch.bfloat16, device=dev)
    _check(v_new, "v_new", torch.bfloat16, device=dev)
    _check(cu_new, "cu_new", torch.int32, B + 1, dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    st = lib.kv_paged_append(ctypes.byref(s), B, _ptr(k_new), _ptr(v_new), _ptr(cu_new), N,
                             _ptr(workspace), workspace.numel(), _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError("kv_paged_append", st)


def kv_rollback(cache: PagedKVCache, num_accepted: torch.Tensor, cu_draft: torch.Tensor,
                draft: bool = False) -> None:
    """Enqueue the rollback of every request to its committed prefix (kv_rollback), or of
    the draft model's cache under the draft's convention (kv_rollback_draft)."""
    lib = load_library()
    dev = cache.device
    B = cu_draft.numel() - 1
    _check(num_accepted, "num_accepted", torch.int32, B, dev)
    _check(cu_draft, "cu_draft", torch.int32, B + 1, dev)
    fn = "kv_rollback_draft" if draft else "kv_rollback"
    st = getattr(lib, fn)(ctypes.byref(cache.struct), B, _ptr(num_accepted), _ptr(cu_draft),
                          _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError(fn, st)


def specdec_cycle_workspace_size(B: int, K: int, V: int, dtype: int, top_k: int,
                                 top_p: float = 1.0, params: Optional[SpecdecParams] = None) -> int:
    return int(load_library().specdec_cycle_workspace_size(B, K, V, dtype, top_k, float(top_p),
                                                           _pref(params)))


def _cycle_args(cache, k_new, v_new, target_logits, draft_logits, draft_tokens, cu_draft,
                u_accept, u_sample, max_k, temperature, top_k, out_tokens, num_accepted,
                num_emitted, err_word, debug, top_p, temperatures, top_ks, top_ps, top_k_max,
                eos_tokens, max_emit):
    """Checked C arguments of a cycle call, up to (not including) the workspace."""
    dev = target_logits.device
    dtype = _logits_dtype(target_logits)
    if target_logits.dim() != 2:
        raise ValueError("target_logits must be [K+B, V]")
    B = cu_draft.numel() - 1
    R, V = target_logits.shape
    K = R - B
    s = cache.struct
    shape = (s.num_layers, K + B, s.num_kv_heads, s.head_dim)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new / v_new must be {shape}")
    _check(k_new, "k_new", torch.bfloat16, device=dev)
    _check(v_new, "v_new", torch.bfloat16, device=dev)
    _check(target_logits, "target_logits", target_logits.dtype, device=dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, K * V, dev)
    _check(draft_tokens, "draft_tokens", torch.int32, K, dev)
    _check(cu_draft, "cu_draft", torch.int32, B + 1, dev)
    _check(u_accept, "u_accept", torch.float32, K, dev)
    _check(u_sample, "u_sample", torch.float32, B, dev)
    _check(out_tokens, "out_tokens", torch.int32, K + B, dev)
    _check(num_accepted, "num_accepted", torch.int32, B, dev)
    _check(num_emitted, "num_emitted", torch.int32, B, dev)
    _check(err_word, "err_word", torch.int32, 1, dev)
    prm = _params(B, dev, temperatures, top_ks, top_ps, top_k_max, eos_tokens, max_emit)
    args = (ctypes.byref(s), _ptr(k_new), _ptr(v_new), _ptr(target_logits), _ptr(draft_logits),
            dtype, _ptr(draft_tokens), _ptr(cu_draft), _ptr(u_accept), _ptr(u_sample), B, K,
            max_k, V, float(temperature), int(top_k), float(top_p), _pref(prm), _ptr(out_tokens),
            _ptr(num_accepted), _ptr(num_emitted), _ptr(err_word),
            ctypes.byref(debug) if debug is not None else None)
    return args, prm, dev


def specdec_cycle(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                  target_logits: torch.Tensor, draft_logits: torch.Tensor,
                  draft_tokens: torch.Tensor, cu_draft: torch.Tensor,
                  u_accept: torch.Tensor, u_sample: torch.Tensor, *, max_k: int,
                  temperature: float, top_k: int, out_tokens: torch.Tensor,
                  num_accepted: torch.Tensor, num_emitted: torch.Tensor,
                  err_word: torch.Tensor, workspace: torch.Tensor,
                  debug: Optional[SpecdecDebug] = None, top_p: float = 1.0,
                  temperatures: Optional[torch.Tensor] = None,
                  top_ks: Optional[torch.Tensor] = None, top_ps: Optional[torch.Tensor] = None,
                  top_k_max: Optional[int] = None, eos_tokens: Optional[torch.Tensor] = None,
                  max_emit: Optional[torch.Tensor] = None, early_exit: bool = False) -> None:
    """Enqueue append -> verify -> rollback of one cycle as fused launches. With
    ``early_exit`` (specdec_cycle_early_exit) the row statistics run position by position and
    no row past a request's first rejection is read."""
    lib = load_library()
    args, prm, dev = _cycle_args(cache, k_new, v_new, target_logits, draft_logits, draft_tokens,
                                 cu_draft, u_accept, u_sample, max_k, temperature, top_k,
                                 out_tokens, num_accepted, num_emitted, err_word, debug, top_p,
                                 temperatures, top_ks, top_ps, top_k_max, eos_tokens, max_emit)
    _check(workspace, "workspace", torch.uint8, None, dev)
    name = "specdec_cycle_early_exit" if early_exit else "specdec_cycle"
    st = getattr(lib, name)(*args, _ptr(workspace), workspace.numel(), _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError(name, st)


def specdec_cycle_static(cache: PagedKVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                         target_logits: torch.Tensor, draft_logits: torch.Tensor,
                         draft_tokens: torch.Tensor, cu_draft: torch.Tensor,
                         u_accept: torch.Tensor, u_sample: torch.Tensor, *, max_k: int,
                         temperature: float, top_k: int, out_tokens: torch.Tensor,
                         num_accepted: torch.Tensor, num_emitted: torch.Tensor,
                         err_word: torch.Tensor, debug: Optional[SpecdecDebug] = None,
                         top_p: float = 1.0, temperatures: Optional[torch.Tensor] = None,
                         top_ks: Optional[torch.Tensor] = None,
                         top_ps: Optional[torch.Tensor] = None, top_k_max: Optional[int] = None,
                         eos_tokens: Optional[torch.Tensor] = None,
                         max_emit: Optional[torch.Tensor] = None) -> None:
    """specdec_cycle over the library's static scratch array (no workspace argument, nothing
    allocated); calls that overlap on one GPU race."""
    lib = load_library()
    args, prm, dev = _cycle_args(cache, k_new, v_new, target_logits, draft_logits, draft_tokens,
                                 cu_draft, u_accept, u_sample, max_k, temperature, top_k,
                                 out_tokens, num_accepted, num_emitted, err_word, debug, top_p,
                                 temperatures, top_ks, top_ps, top_k_max, eos_tokens, max_emit)
    st = lib.specdec_cycle_static(*args, _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError("specdec_cycle_static", st)


def specdec_probe_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Stream src once with the statistics launches' access pattern (bandwidth probe)."""
    lib = load_library()
    st = lib.specdec_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                _stream(src.device))
    if st != SPECDEC_OK:
        raise SpecdecError("specdec_probe_read", st)


def specdec_probe_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """Copy src into dst with the K/V scatter's loads and stores (bandwidth probe)."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("specdec_probe_copy: dst is smaller than src")
    st = lib.specdec_probe_copy(_ptr(dst), _ptr(src), nbytes, _stream(src.device))
    if st != SPECDEC_OK:
        raise SpecdecError("specdec_probe_copy", st)


# --- HIP events and stream waits through the runtime (timing, cross-stream ordering) -----

_hip = None


def _hip_rt() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                               ctypes.c_int]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


_HIP_ATTR_MEMORY_BUS_WIDTH = 59      # hipDeviceAttributeMemoryBusWidth (bits)
_HIP_ATTR_MEMORY_CLOCK_RATE = 60     # hipDeviceAttributeMemoryClockRate (kHz)


def device_memory(device: int = 0) -> dict:
    """The device's memory bus width (bits) and peak memory clock (kHz) as HIP reports
    them, and their product in GB/s (bytes per clock x clock; the transfers per clock
    depend on the memory type)."""
    rt = _hip_rt()
    v = ctypes.c_int()
    out = {}
    for name, attr in (("bus_width_bits", _HIP_ATTR_MEMORY_BUS_WIDTH),
                       ("clock_khz", _HIP_ATTR_MEMORY_CLOCK_RATE)):
        if rt.hipDeviceGetAttribute(ctypes.byref(v), attr, device) != 0:
            raise RuntimeError("hipDeviceGetAttribute failed")
        out[name] = int(v.value)
    out["clock_x_bus_gbps"] = out["clock_khz"] * 1e3 * out["bus_width_bits"] / 8 / 1e9
    return out


class HipEvent:
    """A hipEvent_t; timing=False creates a synchronization-only event."""

    def __init__(self, timing: bool = True):
        self.handle = ctypes.c_void_p()
        flags = 0 if timing else 0x2   # hipEventDisableTiming
        if _hip_rt().hipEventCreateWithFlags(ctypes.byref(self.handle), flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream: "torch.cuda.Stream") -> None:
        if _hip_rt().hipEventRecord(self.handle, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait_on(self, stream: "torch.cuda.Stream") -> None:
        """Make `stream` wait until this event has completed."""
        if _hip_rt().hipStreamWaitEvent(ctypes.c_void_p(stream.cuda_stream), self.handle, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        rt = _hip_rt()
        rt.hipEventSynchronize(end.handle)
        ms = ctypes.c_float()
        if rt.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle:
                _hip_rt().hipEventDestroy(self.handle)
        except Exception:
            pass


def specdec_tree_verify_workspace_size(B: int, N: int, V: int, dtype: int = SPECDEC_BF16,
                                       top_k: int = 0, top_p: float = 1.0,
                                       params: Optional[SpecdecParams] = None) -> int:
    return int(load_library().specdec_tree_verify_workspace_size(B, N, V, dtype, top_k,
                                                                 float(top_p), _pref(params)))


def specdec_tree_verify(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                        tree_tokens: torch.Tensor, tree_parent: torch.Tensor,
                        cu_nodes: torch.Tensor, u_accept: torch.Tensor, u_sample: torch.Tensor,
                        *, max_nodes: int, temperature: float, out_tokens: torch.Tensor,
                        accepted_nodes: torch.Tensor, num_accepted: torch.Tensor,
                        num_emitted: torch.Tensor, err_word: torch.Tensor,
                        workspace: torch.Tensor, req_flags: Optional[torch.Tensor] = None,
                        team: int = 0, top_k: int = 0, top_p: float = 1.0,
                        temperatures: Optional[torch.Tensor] = None,
                        top_ks: Optional[torch.Tensor] = None,
                        top_ps: Optional[torch.Tensor] = None,
                        top_k_max: Optional[int] = None) -> None:
    """Enqueue the verification of one draft tree per request (shapes as in the header);
    ``team`` workgroups share each request's walk (0: automatic); temperatures / top_ks /
    top_ps: optional per-request [B] device tensors replacing the scalars."""
    lib = load_library()
    dev = target_logits.device
    dtype = _logits_dtype(target_logits)
    if target_logits.dim() != 2:
        raise ValueError("target_logits must be [N+B, V]")
    B = cu_nodes.numel() - 1
    R, V = target_logits.shape
    N = R - B
    _check(target_logits, "target_logits", target_logits.dtype, device=dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, R * V, dev)
    _check(tree_tokens, "tree_tokens", torch.int32, N, dev)
    _check(tree_parent, "tree_parent", torch.int32, N, dev)
    _check(cu_nodes, "cu_nodes", torch.int32, B + 1, dev)
    _check(u_accept, "u_accept", torch.float32, N, dev)
    _check(u_sample, "u_sample", torch.float32, B, dev)
    _check(out_tokens, "out_tokens", torch.int32, N + B, dev)
    _check(accepted_nodes, "accepted_nodes", torch.int32, N, dev)
    _check(num_accepted, "num_accepted", torch.int32, B, dev)
    _check(num_emitted, "num_emitted", torch.int32, B, dev)
    _check(err_word, "err_word", torch.int32, 1, dev)
    if req_flags is not None:
        _check(req_flags, "req_flags", torch.int32, B, dev)
    _check(workspace, "workspace", torch.uint8, device=dev)
    prm = _params(B, dev, temperatures, top_ks, top_ps, top_k_max)
    st = lib.specdec_tree_verify(
        _ptr(target_logits), _ptr(draft_logits), dtype, _ptr(tree_tokens), _ptr(tree_parent),
        _ptr(cu_nodes), _ptr(u_accept), _ptr(u_sample), B, N, max_nodes, V, float(temperature),
        int(top_k), float(top_p), _pref(prm), _ptr(out_tokens),
        _ptr(accepted_nodes) if N else None,
        _ptr(num_accepted),
        _ptr(num_emitted),
        _ptr(err_word), _ptr(req_flags) if req_flags is not None else None, int(team),
        _ptr(workspace), workspace.numel(), _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError("specdec_tree_verify", st)


def kv_tree_commit(cache: PagedKVCache, num_accepted: torch.Tensor, accepted_nodes: torch.Tensor,
                   cu_nodes: torch.Tensor) -> None:
    """Enqueue the gather of every request's accepted path and the truncation after it."""
    lib = load_library()
    dev = cache.device
    B = cu_nodes.numel() - 1
    _check(num_accepted, "num_accepted", torch.int32, B, dev)
    _check(cu_nodes, "cu_nodes", torch.int32, B + 1, dev)
    _check(accepted_nodes, "accepted_nodes", torch.int32, None, dev)
    st = lib.kv_tree_commit(ctypes.byref(cache.struct), B, _ptr(num_accepted),
                            _ptr(accepted_nodes) if accepted_nodes.numel() else None,
                            _ptr(cu_nodes), int(accepted_nodes.numel()), _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError("kv_tree_commit", st)


class ContigKVCache:
    """Device tensors of one contiguous cache plus the C struct that points at them."""

    def __init__(self, pool: torch.Tensor, seq_lens: torch.Tensor, state: torch.Tensor):
        if pool.dim() != 6 or pool.dtype != torch.bfloat16 or pool.shape[1] != 2:
            raise ValueError("pool must be bf16 [L][2][batch][max_len][H][D]")
        L, _, Bc, M, H, D = pool.shape
        _check(pool, "pool", torch.bfloat16, device=pool.device)
        _check(seq_lens, "seq_lens", torch.int32, Bc, pool.device)
        _check(state, "state", torch.int32, 1, pool.device)
        self.pool, self.seq_lens, self.state = pool, seq_lens, state
        self.device = pool.device
        self.struct = KvContigCacheStruct(pool.data_ptr(), L, H, D, M, Bc, seq_lens.data_ptr(),
                                          state.data_ptr())


def kv_contig_append(cache: ContigKVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                     cu_new: torch.Tensor) -> None:
    lib = load_library()
    dev = cache.device
    B = cu_new.numel() - 1
    _check(cu_new, "cu_new", torch.int32, B + 1, dev)
    N = k_new.shape[1] if k_new.dim() == 4 else 0
    _check(k_new, "k_new", torch.bfloat16, device=dev)
    _check(v_new, "v_new", torch.bfloat16, device=dev)
    st = lib.kv_contig_append(ctypes.byref(cache.struct), B, _ptr(k_new) if N else None,
                              _ptr(v_new) if N else None, _ptr(cu_new), N, _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError("kv_contig_append", st)


def kv_contig_rollback(cache: ContigKVCache, num_accepted: torch.Tensor, cu_draft: torch.Tensor,
                       draft: bool = False) -> None:
    lib = load_library()
    dev = cache.device
    B = cu_draft.numel() - 1
    _check(num_accepted, "num_accepted", torch.int32, B, dev)
    _check(cu_draft, "cu_draft", torch.int32, B + 1, dev)
    st = lib.kv_contig_rollback(ctypes.byref(cache.struct), B, _ptr(num_accepted), _ptr(cu_draft),
                                1 if draft else 0, _stream(dev))
    if st != SPECDEC_OK:
        raise SpecdecError("kv_contig_rollback", st)
