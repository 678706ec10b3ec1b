"""The C-ABI library loads without a GPU, exports every function include/specdec.h declares,
and rejects bad host-visible arguments before touching the device (no compute calls)."""

import ctypes
import os
import re

import pytest

from rejection_sampling_verify_specdec_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specdec.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("typedef")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libspecdec.so not built: run __graft_entry__.build()")
    return binding.load_library()


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (0, -1, -3, -4, -5, 12345):
        assert isinstance(binding.status_string(st), str) and binding.status_string(st)


def test_workspace_sizes(lib):
    n = binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 0)
    assert n > 0 and n % 256 == 0
    # top-k rows keep per-chunk candidate lists: 2816 rows x 8 chunks x 1040 keys x 4 bytes
    assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 64) >= \
        2816 * 8 * 1040 * 4
    # above the chunked select's top_k limit only the generic select runs: no lists
    assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 2000) < n
    assert binding.specdec_verify_workspace_size(0, 0, 10, 0, 0) == 0
    assert binding.kv_paged_append_workspace_size(512, 3000) >= 16 + 512 * 16 + 3000 * 8
    assert binding.kv_paged_append_workspace_size(0, 10) == 0
    # the largest vocabulary is accepted, one more token is not
    assert binding.specdec_verify_workspace_size(1, 1, binding.MAX_V, binding.SPECDEC_BF16, 64) > 0
    assert binding.specdec_verify_workspace_size(1, 1, binding.MAX_V + 1, binding.SPECDEC_BF16, 0) == 0
    assert binding.specdec_cycle_workspace_size(1, 1, binding.MAX_V + 1, binding.SPECDEC_F32, 0) == 0
    # per-request parameters: lists for the largest chunk k, row parameters, chunk partials
    pr = binding.SpecdecParams(16, 16, None, 64)
    assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 0, 1.0,
                                                 pr) >= 2816 * 8 * 1040 * 4 + 2816 * 16
    assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 0, 1.0,
                                                 binding.SpecdecParams(None, 16, None, -1)) == 0
    assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 0, 1.0,
                                                 binding.SpecdecParams(None, None, None, 0)) == n
    # top-p alone gathers candidates like top-k; top-p NaN is rejected, <= 0 or >= 1 is off
    assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 0,
                                                 0.9) >= 2816 * 8 * 1040 * 4
    assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 0,
                                                 float("nan")) == 0
    for off in (0.0, -1.0, 1.0, 2.0):
        assert binding.specdec_verify_workspace_size(256, 1280, 128256, binding.SPECDEC_BF16, 0,
                                                     off) == n


def test_host_validation_returns_einval_without_gpu(lib):
    vp = None
    # B = 0
    assert lib.specdec_verify(vp, vp, 1, vp, vp, vp, vp, 0, 0, 4, 10, 1.0, 0, 1.0, None, vp, vp, vp, vp,
                              None, vp, 0, vp) == binding.SPECDEC_EINVAL
    # temperature <= 0, and NaN
    for T in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.specdec_verify(1, 1, 1, 1, 1, 1, 1, 1, 1, 4, 10, T, 0, 1.0, None, 1, 1, 1, 1,
                                  None, 16, 1 << 30, vp) == binding.SPECDEC_EINVAL
    # top_p NaN
    assert lib.specdec_verify(1, 1, 1, 1, 1, 1, 1, 1, 1, 4, 10, 1.0, 0, float("nan"), None, 1, 1, 1, 1,
                              None, 16, 1 << 30, vp) == binding.SPECDEC_EINVAL
    # per-request arrays: T and top_p scalars they replace are not checked; top_k_max < 0
    pr_t = binding.SpecdecParams(16, None, None, 0)
    assert lib.specdec_verify(1, 1, 1, 1, 1, 1, 1, 1, 1, 4, 10, float("nan"), 0, 1.0,
                              ctypes.byref(pr_t), 1, 1, 1, 1, None, 16, 8,
                              vp) == binding.SPECDEC_EWORKSPACE
    pr_k = binding.SpecdecParams(None, 16, None, -1)
    assert lib.specdec_verify(1, 1, 1, 1, 1, 1, 1, 1, 1, 4, 10, 1.0, 0, 1.0, ctypes.byref(pr_k),
                              1, 1, 1, 1, None, 16, 1 << 30, vp) == binding.SPECDEC_EINVAL
    # max_k above the limit, K > B * max_k, bad dtype
    assert lib.specdec_verify(1, 1, 1, 1, 1, 1, 1, 1, 1, 65, 10, 1.0, 0, 1.0, None, 1, 1, 1, 1,
                              None, 16, 1 << 30, vp) == binding.SPECDEC_EINVAL
    assert lib.specdec_verify(1, 1, 1, 1, 1, 1, 1, 2, 9, 4, 10, 1.0, 0, 1.0, None, 1, 1, 1, 1,
                              None, 16, 1 << 30, vp) == binding.SPECDEC_EINVAL
    assert lib.specdec_verify(1, 1, 7, 1, 1, 1, 1, 1, 1, 4, 10, 1.0, 0, 1.0, None, 1, 1, 1, 1,
                              None, 16, 1 << 30, vp) == binding.SPECDEC_EINVAL
    # workspace too small / misaligned
    assert lib.specdec_verify(16, 16, 1, 16, 16, 16, 16, 1, 1, 4, 10, 1.0, 0, 1.0, None, 16, 16, 16, 16,
                              None, 16, 8, vp) == binding.SPECDEC_EWORKSPACE
    assert lib.specdec_verify(16, 16, 1, 16, 16, 16, 16, 1, 1, 4, 10, 1.0, 0, 1.0, None, 16, 16, 16, 16,
                              None, 17, 1 << 30, vp) == binding.SPECDEC_EWORKSPACE


def test_kv_host_validation_without_gpu(lib):
    c = binding.KvPagedCacheStruct(16, 2, 2, 8, 16, 64, 8, 16, 16, 16, 16, 16, 16)
    assert lib.kv_rollback(ctypes.byref(c), 0, 16, 16, None) == binding.SPECDEC_EINVAL
    assert lib.kv_rollback(ctypes.byref(c), 4097, 16, 16, None) == binding.SPECDEC_EINVAL
    bad = binding.KvPagedCacheStruct(16, 2, 1, 3, 16, 64, 8, 16, 16, 16, 16, 16, 16)  # H*D*2=6
    assert lib.kv_rollback(ctypes.byref(bad), 4, 16, 16, None) == binding.SPECDEC_EINVAL
    assert lib.kv_paged_append(ctypes.byref(c), 4, 16, 16, 16, -1, 16, 1 << 20,
                               None) == binding.SPECDEC_EINVAL
    assert lib.kv_paged_append(ctypes.byref(c), 4, 16, 16, 16, 8, 16, 8,
                               None) == binding.SPECDEC_EWORKSPACE
    nopool = binding.KvPagedCacheStruct(None, 2, 2, 8, 16, 64, 8, 16, 16, 16, 16, 16, 16)
    assert lib.kv_paged_append(ctypes.byref(nopool), 4, 16, 16, 16, 8, 16, 1 << 20,
                               None) == binding.SPECDEC_EINVAL


def test_product_path_fails_loudly_without_library(tmp_path):
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            binding.load_library(str(tmp_path / "nope.so"))
    finally:
        binding._lib = saved


def test_tree_workspace_and_host_validation_without_gpu(lib):
    # the pass ring: (N + 2B) slots of 4 doubles per 2048-token sub-chunk, after the counters
    n = binding.specdec_tree_verify_workspace_size(128, 2071, 128256)
    assert n >= (2071 + 256) * 4 * 63 * 8 + 128 * 64 * 4
    assert binding.specdec_tree_verify_workspace_size(0, 0, 100) == 0
    assert binding.specdec_tree_verify_workspace_size(1, 0, binding.MAX_V + 1) == 0
    assert binding.specdec_tree_verify_workspace_size(1, 0, 100, dtype=7) == 0
    assert binding.specdec_tree_verify_workspace_size(1, 0, 100, top_p=float("nan")) == 0
    # top-k / top-p add every row's statistics, threshold and select lists
    R = 2 * (2071 + 128)
    for tk, tp in ((64, 1.0), (0, 0.9), (50, 0.9), (2000, 1.0)):
        m = binding.specdec_tree_verify_workspace_size(128, 2071, 128256, binding.SPECDEC_BF16,
                                                       tk, tp)
        assert m >= n + R * (16 + 4)
    # off: top_k 0 or >= V, top_p >= 1 or <= 0
    for tk, tp in ((0, 1.0), (128256, 1.0), (0, 0.0), (-3, 1.5)):
        assert binding.specdec_tree_verify_workspace_size(128, 2071, 128256,
                                                          binding.SPECDEC_BF16, tk, tp) == n
    vp = None

    def call(team=0, ws=16, nbytes=1 << 30, T=1.0, B=1, N=1, max_nodes=4, V=1000, top_k=0,
             top_p=1.0, pr=None):
        return lib.specdec_tree_verify(16, 16, binding.SPECDEC_BF16, 16, 16, 16, 16, 16, B, N,
                                       max_nodes, V, T, top_k, top_p,
                                       ctypes.byref(pr) if pr is not None else None, 16, 16,
                                       16, 16, 16, vp, team, ws, nbytes, vp)
    assert call(team=-1) == binding.SPECDEC_EINVAL
    assert call(team=binding.MAX_TREE_TEAM + 1) == binding.SPECDEC_EINVAL
    assert call(T=0.0) == binding.SPECDEC_EINVAL
    assert call(top_p=float("nan")) == binding.SPECDEC_EINVAL
    assert call(max_nodes=binding.MAX_TREE + 1) == binding.SPECDEC_EINVAL
    assert call(N=5, max_nodes=4) == binding.SPECDEC_EINVAL
    assert call(ws=None) == binding.SPECDEC_EWORKSPACE
    assert call(ws=17) == binding.SPECDEC_EWORKSPACE
    assert call(nbytes=binding.specdec_tree_verify_workspace_size(1, 1, 1000) - 1,
                team=1) == binding.SPECDEC_EWORKSPACE
    need = binding.specdec_tree_verify_workspace_size(1, 1, 1000, binding.SPECDEC_BF16, 8, 0.9)
    assert call(nbytes=need - 1, team=1, top_k=8, top_p=0.9) == binding.SPECDEC_EWORKSPACE
    # per-request arrays: they replace the scalars (a bad scalar is then not checked);
    # stopping arrays are not taken on trees; a top_k array needs top_k_max >= 0
    P = binding.SpecdecParams
    temps = P(16, None, None, 0, None, None)
    assert call(T=0.0, pr=temps, nbytes=8, team=1) == binding.SPECDEC_EWORKSPACE
    assert call(top_p=float("nan"), pr=P(None, None, 16, 0, None, None), nbytes=8,
                team=1) == binding.SPECDEC_EWORKSPACE
    assert call(pr=P(None, None, None, 0, 16, None)) == binding.SPECDEC_EINVAL
    assert call(pr=P(None, None, None, 0, None, 16)) == binding.SPECDEC_EINVAL
    assert call(pr=P(None, 16, None, -1, None, None)) == binding.SPECDEC_EINVAL
    size = lambda pr: lib.specdec_tree_verify_workspace_size(128, 2071, 128256,
                                                             binding.SPECDEC_BF16, 0, 1.0,
                                                             ctypes.byref(pr))
    assert size(temps) > n                          # each row's parameters
    assert size(P(None, 16, None, 64, None, None)) > size(temps)   # and the select
    assert size(P(None, None, None, 0, 16, None)) == 0


def test_early_exit_host_validation_without_gpu(lib):
    # the early-exit cycle takes every transform (temperature, top-k, top-p, scalar or per
    # request); the acceptance analytics are EINVAL before anything is enqueued; allowed
    # arguments go on to the workspace check (8 bytes: EWORKSPACE), as specdec_cycle does
    c = binding.KvPagedCacheStruct(16, 2, 2, 8, 16, 64, 8, 16, 16, 16, 16, 16, 16)

    def call(fn, top_k=0, top_p=1.0, pr=None, dbg=None):
        return fn(ctypes.byref(c), 16, 16, 16, 16, 1, 16, 16, 16, 16, 4, 8, 2, 1000, 1.0, top_k,
                  top_p, ctypes.byref(pr) if pr is not None else None, 16, 16, 16, 16,
                  ctypes.byref(dbg) if dbg is not None else None, 16, 8, None)

    ee, full = lib.specdec_cycle_early_exit, lib.specdec_cycle
    analytics = binding.SpecdecDebug()
    analytics.accept_prob = 16
    eos_only = binding.SpecdecParams(None, None, None, 0, 16, 16)
    assert call(ee, dbg=analytics) == binding.SPECDEC_EINVAL
    assert call(full, dbg=analytics) == binding.SPECDEC_EWORKSPACE
    for kw in (dict(), dict(top_k=1000), dict(top_k=0, top_p=1.0, pr=eos_only),
               dict(pr=binding.SpecdecParams(16, None, None, 0)),   # temperature array
               dict(top_k=10), dict(top_p=0.9), dict(top_p=0.5, top_k=999),
               dict(pr=binding.SpecdecParams(None, 16, None, 4)),
               dict(pr=binding.SpecdecParams(None, None, 16, 0)),
               dict(dbg=binding.SpecdecDebug())):
        assert call(ee, **kw) == binding.SPECDEC_EWORKSPACE, kw
    # the checks both entry points share
    assert call(ee, top_p=float("nan")) == binding.SPECDEC_EINVAL
    assert ee(ctypes.byref(c), 16, 16, 16, 16, 1, 16, 16, 16, 16, 0, 8, 2, 1000, 1.0, 0, 1.0,
              None, 16, 16, 16, 16, None, 16, 1 << 30, None) == binding.SPECDEC_EINVAL


def test_verify_early_exit_host_validation_without_gpu(lib):
    # as the cycle's: every transform, no analytics; allowed arguments reach the workspace
    # check
    def call(fn, top_k=0, top_p=1.0, pr=None, dbg=None):
        return fn(16, 16, 1, 16, 16, 16, 16, 4, 8, 2, 1000, 1.0, top_k, top_p,
                  ctypes.byref(pr) if pr is not None else None, 16, 16, 16, 16,
                  ctypes.byref(dbg) if dbg is not None else None, 16, 8, None)

    ee, full = lib.specdec_verify_early_exit, lib.specdec_verify
    analytics = binding.SpecdecDebug()
    analytics.expected_emitted = 16
    assert call(ee, dbg=analytics) == binding.SPECDEC_EINVAL
    assert call(full, dbg=analytics) == binding.SPECDEC_EWORKSPACE
    for kw in (dict(), dict(top_k=1000), dict(pr=binding.SpecdecParams(16, None, None, 0)),
               dict(top_k=10), dict(top_p=0.9), dict(pr=binding.SpecdecParams(None, None, 16, 0)),
               dict(pr=binding.SpecdecParams(None, 16, None, 4))):
        assert call(ee, **kw) == binding.SPECDEC_EWORKSPACE, kw


def test_static_cycle_refuses_calls_larger_than_its_scratch(lib):
    # the size check comes before anything touches a device: a full top-k batch needs more
    # than the static array and is refused with SPECDEC_ESCRATCH, here without a GPU
    need = binding.specdec_cycle_workspace_size(128, 1024, 128256, binding.SPECDEC_BF16, 64)
    assert need > binding.STATIC_SCRATCH_BYTES
    st = lib.specdec_cycle_static(None, None, None, None, None, binding.SPECDEC_BF16, None, None,
                                  None, None, 128, 1024, 8, 128256, 0.8, 64, 1.0, None, None,
                                  None, None, None, None, None)
    assert st == binding.SPECDEC_ESCRATCH
    assert "static" in binding.status_string(st)


def test_the_library_loaded_is_the_one_asked_for(lib):
    # under the host-sanitizer test, SPECDEC_LIBRARY names the sanitized build
    want = os.environ.get("SPECDEC_LIBRARY")
    if want:
        assert os.path.samefile(lib._name, want)
        data = open(want, "rb").read().decode("latin-1")
        assert "__asan_init" in data and "__ubsan_handle" in data


def test_probe_host_validation_without_gpu(lib):
    # the bandwidth probes refuse null, misaligned, empty, ragged and overlapping buffers
    # before anything is enqueued
    E = binding.SPECDEC_EINVAL
    assert lib.specdec_probe_read(None, 1 << 20, 4096, None) == E
    assert lib.specdec_probe_read(4096, 1 << 20, None, None) == E
    assert lib.specdec_probe_read(4100, 1 << 20, 8, None) == E
    assert lib.specdec_probe_read(4096, 0, 8, None) == E
    assert lib.specdec_probe_read(4096, 1000, 8, None) == E
    assert lib.specdec_probe_copy(1 << 30, 4096, 0, None) == E
    assert lib.specdec_probe_copy(4096 + (1 << 19), 4096, 1 << 20, None) == E
    assert lib.specdec_probe_copy(4096, 4096 + (1 << 19), 1 << 20, None) == E
    assert lib.specdec_probe_copy(4104, 1 << 30, 1 << 20, None) == E
