"""Benchmark: one speculative cycle (paged append -> verify -> rollback) per step.

Default workload: B=256 requests, k=5 proposals, V=128256, bf16 logits (target N(0,3),
draft = target + N(0,1.5)), T=0.7, paged KV of 32 layers x 8 KV heads x 128 bf16 with
16-slot blocks and prefix lengths U[512,4096]. Inputs are synthetic, seeded and resident
in HBM before timing. Steps run back to back on one stream; the cache grows by 1 + a_b
per request per step, as in steady-state decoding.

Prints one JSON line with the throughput (verified draft positions per second), the
achieved HBM bandwidth of the whole cycle and, under "roofline", of the row-statistics
kernel (timed with HIP events recorded around it inside the timed steps), plus a CPU
baseline: the fp64 oracle timed on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from rejection_sampling_verify_specdec_amd.profsum import source_hash  # noqa: E402

METRIC = "verified draft positions/sec + achieved HBM GB/s (% peak), B=256 k=5 V=128256 bf16"
PEAK_GBPS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30,
                   help="untimed cycles before the timed ones")
    p.add_argument("--settle-ms", type=float, default=150.0,
                   help="before the warm-up: run cycles for this long (restoring the cache "
                        "metadata every 16 of them, so the cache the warm-up and timed cycles "
                        "see is unchanged) while the GPU's clocks rise under load")
    p.add_argument("--workload", default="c2")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--batch", type=int, default=None,
                   help="override the workload's batch size B (latency at small batches)")
    p.add_argument("--top-k", type=int, default=None,
                   help="override the workload's top_k (0 = off)")
    p.add_argument("--top-p", type=float, default=1.0,
                   help="nucleus mass after temperature and top-k (<= 0 or >= 1 = off)")
    p.add_argument("--per-request", action="store_true",
                   help="pass the transform as per-request arrays (same values for every "
                        "request): measures the per-request path")
    p.add_argument("--schedule", choices=["fused", "early-exit", "serial", "overlap"], default="fused",
                   help="fused: specdec_cycle (allocation inside the logit-streaming launch, "
                        "K/V scatter beside the sampling workgroups); serial: append, verify, "
                        "rollback as three calls on one stream; overlap: the three calls with "
                        "the append on a second stream after the logit rows are streamed; "
                        "early-exit: specdec_cycle_early_exit (row statistics position by "
                        "position, no row read past a request's first rejection)")
    p.add_argument("--timing-every", type=int, default=10,
                   help="attach HIP timing events to the row-statistics launch of every "
                        "n-th step (they add a few microseconds to those steps)")
    p.add_argument("--team", type=int, default=0,
                   help="tree workloads: workgroups per request walk (0: automatic)")
    p.add_argument("--flush-mib", type=int, default=512,
                   help="for the flushed percentiles: MiB written before each of those cycles, "
                        "outside its events, so no input is left in the 256 MB MALL (0: skip)")
    p.add_argument("--graph", action="store_true",
                   help="also time the fused cycle captured once in a HIP graph and replayed "
                        "(no host launch cost per cycle: what small batches need)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-early-exit-compare", action="store_true",
                   help="skip timing specdec_cycle_early_exit beside the fused cycle")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the read / copy bandwidth probes after the timed region")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="run one plain device-to-device copy of this many MiB before timing "
                        "(a known-size reference for HBM traffic counters)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time the oracle baseline runs for")
    p.add_argument("--cpu-workers", type=int, default=0,
                   help="processes for the n-core oracle baseline (0: min(16, available))")
    return p.parse_args()


def probe_ceilings(binding, torch, d, srcs, copy_mib: int, reps: int = 20):
    """This device's read and copy ceilings from the library's bandwidth probes, measured
    after the timed region: the tensors in srcs (the logit rows; at least copy_mib MiB)
    streamed reps times with the statistics launches' access pattern, and a copy_mib MiB
    buffer copied reps times with the fastest copy shape measured on this part; events
    around each group of launches."""
    sink = torch.zeros(1, dtype=torch.int32, device=d)
    # whole 16-byte vectors of each tensor (the probes' unit); small batches' rows are too
    # few to keep the device busy, so below copy_mib MiB a buffer of that size is read
    srcs = [t.reshape(-1).view(torch.uint8) for t in srcs]
    srcs = [t[: t.numel() // 16 * 16] for t in srcs]
    if sum(t.numel() for t in srcs) < copy_mib << 20:
        srcs = [torch.ones(copy_mib << 20, dtype=torch.uint8, device=d)]
    nb_read = sum(t.numel() for t in srcs)

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    t_read = timed(lambda: [binding.specdec_probe_read(t, sink) for t in srcs])
    a = torch.empty(copy_mib << 20, dtype=torch.uint8, device=d).fill_(1)
    b = torch.empty_like(a)
    t_copy = timed(lambda: binding.specdec_probe_copy(b, a))
    nb_copy = 2 * a.numel()
    del a, b
    return {"read_gbps": nb_read / t_read / 1e9, "read_bytes": nb_read,
            "copy_gbps": nb_copy / t_copy / 1e9, "copy_bytes_read_and_written": nb_copy,
            "kernels": "k_probe_read, k_probe_copy", "reps": reps}


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    try:
        d = json.load(open(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")))
    except Exception:
        return None
    if d.get("source_sha256_16") != source_hash():
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(vin, kv, min_seconds: float, top_p: float):
    """The oracle as it stands, one core: whole cycles of the same workload (verify of every
    request, then the paged append and rollback), repeated until min_seconds have passed."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    import oracle
    reps, t_verify, t_kv = 0, 0.0, 0.0
    while reps == 0 or t_verify + t_kv < min_seconds:
        t0 = time.perf_counter()
        res = oracle.verify_batch(vin.target, vin.draft, vin.draft_tokens, vin.cu_draft,
                                  vin.u_accept, vin.u_sample, vin.T, vin.top_k, vin.max_k,
                                  vin.dtype, keep_probs=False, top_p=top_p)
        t1 = time.perf_counter()
        o = oracle.PagedKV(kv.L, kv.H, kv.D, kv.block_size, kv.num_blocks, kv.block_tables,
                           kv.seq_lens, kv.refcount, kv.free_list, kv.free_count, kv.blocks)
        t2 = time.perf_counter()
        o.append(kv.k_new, kv.v_new, kv.cu_new)
        o.rollback(np.where(res.num_accepted >= 0, res.num_accepted, 0), vin.cu_draft)
        t3 = time.perf_counter()
        t_verify += t1 - t0
        t_kv += t3 - t2
        reps += 1
    t = t_verify + t_kv
    return {"value": vin.K * reps / t, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": (f"{reps} whole cycles of the workload ({vin.K} positions each): fp64 "
                       f"verify {t_verify:.2f} s + paged append/rollback {t_kv:.2f} s, "
                       f"input generation and copies excluded")}


def _oracle_shard(path, reqs, T, top_k, max_k, dtype, top_p):
    """One worker of the n-core baseline: verify its requests from memory-mapped inputs."""
    import oracle
    a = {k: np.load(os.path.join(path, k + ".npy"), mmap_mode="r")
         for k in ("target", "draft", "tokens", "cu", "u_acc", "u_smp")}
    t0 = time.perf_counter()
    oracle.verify_batch(a["target"], a["draft"], a["tokens"], a["cu"], a["u_acc"], a["u_smp"], T,
                        top_k, max_k, dtype, requests=reqs, keep_probs=False, top_p=top_p)
    return time.perf_counter() - t0


def cpu_baseline_ncores(vin, top_p: float, workers: int, min_seconds: float = 2.0):
    """The oracle's verification sharded by request over a pool of fresh processes (one
    thread each), inputs memory-mapped from a temporary directory; whole batches repeated
    for at least min_seconds of wall time. The paged append / rollback (sequential by
    definition, and ~2% of the one-core time) are left out of this figure."""
    import multiprocessing as mp
    import tempfile
    with tempfile.TemporaryDirectory(dir="/tmp") as path:
        for k, x in (("target", vin.target), ("draft", vin.draft), ("tokens", vin.draft_tokens),
                     ("cu", vin.cu_draft), ("u_acc", vin.u_accept), ("u_smp", vin.u_sample)):
            np.save(os.path.join(path, k + ".npy"), np.ascontiguousarray(x))
        shards = [list(range(w, vin.B, workers)) for w in range(workers)]
        env = {"OMP_NUM_THREADS": "1", "OPENBLAS_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}
        old = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        try:
            with mp.get_context("spawn").Pool(workers) as pool:
                pool.starmap(_oracle_shard, [(path, [0], vin.T, vin.top_k, vin.max_k, vin.dtype,
                                              top_p)] * workers)        # warm the workers
                reps, t = 0, 0.0
                while reps == 0 or t < min_seconds:
                    t0 = time.perf_counter()
                    pool.starmap(_oracle_shard, [(path, sh, vin.T, vin.top_k, vin.max_k,
                                                  vin.dtype, top_p) for sh in shards])
                    t += time.perf_counter() - t0
                    reps += 1
        finally:
            for k, v in old.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    return {"value": vin.K * reps / t, "unit": "positions/s", "cores": workers, "kind": "oracle",
            "sample": (f"{reps} verifications of the whole batch ({vin.K} positions), requests "
                       f"spread over {workers} processes; paged append / rollback excluded")}


def early_exit_rows(kb, ab, seq):
    """Logit rows the early-exit cycle reads: position by position up to each request's first
    rejection j (= a_b, or k_b when every proposal is accepted) among positions 0 .. seq - 1,
    then, for a request whose first seq proposals were all accepted, every later row in one
    launch. A position p < k_b has a target and a draft row; position k_b the bonus row."""
    rows = 0
    for k, a in zip(kb.tolist(), ab.tolist()):
        j = min(a, k)
        per = lambda p: 2 if p < k else 1
        rows += sum(per(p) for p in range(min(j, seq - 1) + 1))
        if j >= seq:
            rows += sum(per(p) for p in range(seq, k + 1))
    return rows


def acceptance_stats(binding, torch, d, vin, tgt, dft, tokens, cu, u_acc, u_smp, out, nacc,
                     nemit, err, ws, top_p, pr, cycle_ms):
    """After the timed cycles, outside them: verification of the same batch with the
    acceptance analytics on. Reports the mean acceptance probability of a proposal, E[A]
    (expected tokens per cycle and request, the correction or bonus included), the tokens
    this batch actually emitted, and E[A] summed over the batch per second of measured
    cycle time: the section 4 throughput proxy with the draft cost left out (the draft
    model is not part of this path), so an upper bound. Also the analytics pass's cost."""
    B, K = vin.B, vin.K
    beta = torch.empty(max(K, 1), dtype=torch.float64, device=d)
    expd = torch.empty(B, dtype=torch.float64, device=d)
    dbg = binding.SpecdecDebug()
    dbg.accept_prob, dbg.expected_emitted = beta.data_ptr(), expd.data_ptr()

    def call(debug):
        binding.specdec_verify(tgt, dft, tokens, cu, u_acc, u_smp, max_k=vin.max_k,
                               temperature=vin.T, top_k=vin.top_k, out_tokens=out,
                               num_accepted=nacc, num_emitted=nemit, err_word=err, workspace=ws,
                               debug=debug, top_p=top_p, **pr)

    times = {}
    for name, debug in (("plain", None), ("analytics", dbg)):
        for _ in range(3):
            call(debug)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            call(debug)
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / 10
    b = beta[:K].cpu().numpy()
    e = expd.cpu().numpy()
    emitted = nemit.cpu().numpy()
    ok = ~np.isnan(e)
    return {"mean_accept_prob": float(np.nanmean(b)) if K else None,
            "mean_expected_emitted": float(e[ok].mean()) if ok.any() else None,
            "realized_emitted_per_request": float(emitted.mean()),
            "proxy_tokens_per_s_no_draft_cost": float(e[ok].sum() / (cycle_ms / 1e3)),
            "verify_ms": times["plain"], "verify_with_analytics_ms": times["analytics"]}


def tree_main(args):
    """Draft trees: per step, append the pending token and every node (kv_paged_append),
    verify the trees (specdec_tree_verify), keep the accepted paths (kv_tree_commit). The
    line reports verified nodes per second, each call's time from events around it on
    every timed step, and the bytes the walk read, replayed on the host from the outputs
    (per visited position: its max / exp-sum pass, one pass over the row pair per rejected
    child, the bonus pass at a leaf; the draw's rescans of 2048 tokens)."""
    import torch
    from rejection_sampling_verify_specdec_amd import binding, synth

    if not os.path.exists(binding.LIB_PATH):
        from rejection_sampling_verify_specdec_amd import build as _b
        _b.build()
    binding.load_library()
    d = torch.device("cuda:0")
    cfg = dict(synth.TREE_WORKLOADS[args.workload])
    top_k = args.top_k or 0
    top_p = args.top_p
    if args.batch:
        cfg["B"] = args.batch
    print(f"# {args.workload}: drawing the synthetic trees", file=sys.stderr, flush=True)
    tin = synth.make_tree(seed=args.seed, top_k=top_k, **cfg)
    kv = synth.make_kv("c2", tin, seed=args.seed, cycles=args.warmup + args.steps + 2)
    print(f"# {args.workload}: inputs ready, timing", file=sys.stderr, flush=True)
    B, N, V = tin.B, tin.N, tin.V

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(d)

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(d)

    tgt, dft = bf(tin.target), bf(tin.draft)
    tokens, parent, cu = t(tin.tokens), t(tin.parent), t(tin.cu_nodes)
    u_acc, u_smp = t(tin.u_accept), t(tin.u_sample)
    pool = torch.empty((kv.L, 2, kv.num_blocks, kv.block_size, kv.H, kv.D), dtype=torch.bfloat16,
                       device=d)
    if kv.blocks:
        ids = sorted(kv.blocks)
        pool[:, :, torch.tensor(ids, device=d)] = bf(np.stack([kv.blocks[X][0] for X in ids], axis=2))
    cache = binding.PagedKVCache(pool, t(kv.block_tables), t(kv.seq_lens), t(kv.refcount),
                                 t(kv.free_list), torch.tensor([kv.free_count], dtype=torch.int32, device=d),
                                 torch.zeros(1, dtype=torch.int32, device=d))
    k_new, v_new, cu_new = bf(kv.k_new), bf(kv.v_new), t(kv.cu_new)
    out = torch.empty(N + B, dtype=torch.int32, device=d)
    nodes = torch.empty(N, dtype=torch.int32, device=d)
    nacc = torch.empty(B, dtype=torch.int32, device=d)
    nemit = torch.empty(B, dtype=torch.int32, device=d)
    err = torch.zeros(1, dtype=torch.int32, device=d)
    kws = torch.empty(binding.kv_paged_append_workspace_size(B, N + B), dtype=torch.uint8, device=d)
    tws = torch.empty(binding.specdec_tree_verify_workspace_size(B, N, tin.V, binding.SPECDEC_BF16,
                                                                 top_k, top_p),
                      dtype=torch.uint8, device=d)
    n = args.warmup + args.steps
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in range(args.warmup, n)}

    def step(i):
        e = ev.get(i)
        if e:
            e[0].record()
        binding.kv_paged_append(cache, k_new, v_new, cu_new, kws)
        if e:
            e[1].record()
        binding.specdec_tree_verify(tgt, dft, tokens, parent, cu, u_acc, u_smp,
                                    max_nodes=tin.max_nodes, temperature=tin.T, out_tokens=out,
                                    accepted_nodes=nodes, num_accepted=nacc, num_emitted=nemit,
                                    err_word=err, workspace=tws, team=args.team, top_k=top_k,
                                    top_p=top_p)
        if e:
            e[2].record()
        binding.kv_tree_commit(cache, nacc, nodes, cu)
        if e:
            e[3].record()

    if args.settle_ms > 0:
        # clocks rise over tens of milliseconds of load; the cycles run here leave no trace
        # in the cache state (its metadata is restored after every 16)
        c = cache
        meta = (c.block_tables, c.seq_lens, c.refcount, c.free_list, c.free_count, c.state)
        snap = [x.clone() for x in meta]
        err0 = err.clone()
        ts = time.perf_counter()
        while (time.perf_counter() - ts) * 1e3 < args.settle_ms:
            for _ in range(16):
                step(-1)
            for dst, src in zip(meta, snap):
                dst.copy_(src)
            torch.cuda.synchronize()
        err.copy_(err0)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, n):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = lambda a, b: float(np.mean([ev[i][a].elapsed_time(ev[i][b]) for i in ev]))
    append_ms, verify_ms, commit_ms = ms(0, 1), ms(1, 2), ms(2, 3)
    # bytes the walk read, replayed from the outputs
    a = nacc.cpu().numpy()
    path = nodes.cpu().numpy()
    row = V * 2
    filt = 0 < top_k < V or 0 < top_p < 1
    # top-k / top-p: the select reads every target row and the draft row of every position
    # with children once, and the walk takes each position's statistics from it instead of
    # its own pass
    inner = sum(len({int(x) for x in tin.parent[int(tin.cu_nodes[b]):int(tin.cu_nodes[b + 1])]})
                for b in range(B))
    select_bytes = (N + B + inner) * row
    walk = select_bytes if filt else 0
    stats = 0 if filt else 1
    for b in range(B):
        lo, hi = int(tin.cu_nodes[b]), int(tin.cu_nodes[b + 1])
        par = tin.parent[lo:hi]
        kids = [[] for _ in range(hi - lo + 1)]
        for j, pa in enumerate(par):
            kids[int(pa) + 1].append(j)
        v = 0
        steps = list(path[lo: lo + max(int(a[b]), 0)]) + [None]
        for nxt in steps:
            if not kids[v]:
                walk += (stats + 1) * row                         # stats + bonus pass
                break
            walk += stats * 2 * row                               # target + draft stats
            rej = kids[v].index(nxt) if nxt is not None else len(kids[v])
            walk += rej * 2 * row                                 # residual passes
            if nxt is None:
                break
            v = int(nxt) + 1
    res = {
        "metric": "verified draft-tree nodes/sec (tree workload; the headline line is the "
                  "linear cycle)",
        "value": N * args.steps / elapsed,
        "unit": "nodes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{args.workload}: B={B} trees of U{{{cfg['n_range'][0]}.."
                                f"{cfg['n_range'][1]}}} nodes (N={N}), V={V} bf16 T={tin.T:g}"
                                + (f" top_k={top_k}" if 0 < top_k < V else "")
                                + (f" top_p={top_p:g}" if 0 < top_p < 1 else "") + "; "
                                f"paged KV {kv.L}x{kv.H}x{kv.D} bf16, block {kv.block_size}"),
                   "global_batch": B, "parallelism": "single GPU"},
        "tree": {"team": args.team or "auto", "append_ms": append_ms, "verify_ms": verify_ms,
                 "commit_ms": commit_ms,
                 "mean_accepted": float(a[a >= 0].mean()), "walk_bytes": walk,
                 "walk_gbps": walk / (verify_ms / 1e3) / 1e9,
                 "walk_frac_of_peak": walk / (verify_ms / 1e3) / 1e9 / PEAK_GBPS},
    }
    if filt:
        res["tree"]["select_bytes"] = select_bytes
        res["tree"]["walk_bytes_note"] = (
            "select_bytes plus a full row pair per rejected child and a row per bonus: an "
            "upper bound, since a bf16 target row whose kept tokens are listed (up to 512) "
            "is summed over the list instead of re-read")
    if int(cache.state.item()):
        print(f"# warning: cache state word {int(cache.state.item()):#x}", file=sys.stderr)
    print(json.dumps(res))


def main():
    args = parse()
    if args.workload.startswith("t") and args.workload != "tiny":
        if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
            print("bench.py measures one GPU.", file=sys.stderr)
            sys.exit(2)
        return tree_main(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification path shards by request with no "
              "cross-GPU exchange, and runs on more than one GPU are not part of this build.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from rejection_sampling_verify_specdec_amd import binding, synth

    if not os.path.exists(binding.LIB_PATH):
        from rejection_sampling_verify_specdec_amd import build as _b
        _b.build()
    binding.load_library()
    d = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    vin = synth.make_verify(wl, seed=args.seed, B=args.batch,
                            **({} if args.top_k is None else {"top_k": args.top_k}))
    top_p = args.top_p
    # the fused cycle is also timed in its early-exit form, on the same batch and cache,
    # after the timed region
    compare_early = args.schedule == "fused" and not args.no_early_exit_compare
    # the pool holds the warm-up, the timed cycles and twice as many again for the
    # percentiles (without and with a cache flush before each cycle), and the early-exit
    # comparison's cycles
    kv = synth.make_kv(wl, vin, seed=args.seed,
                       cycles=args.warmup + (5 if args.graph else 3) * args.steps + 4 +
                       (args.steps + 10 if compare_early else 0))
    print(f"# inputs drawn in {time.time() - t0:.1f} s: B={vin.B} K={vin.K} V={vin.V} "
          f"NB={kv.num_blocks}", file=sys.stderr, flush=True)

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(d)

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(d)

    logits = bf if vin.dtype == "bf16" else (lambda x: t(x.astype(np.float32)))
    tgt, dft = logits(vin.target), logits(vin.draft)
    tokens, cu = t(vin.draft_tokens), t(vin.cu_draft)
    u_acc, u_smp = t(vin.u_accept), t(vin.u_sample)
    pool_bytes = kv.L * 2 * kv.num_blocks * kv.block_size * kv.H * kv.D * 2
    free_bytes = torch.cuda.mem_get_info(d)[0]
    if pool_bytes > free_bytes:
        sys.exit(f"bench.py: the paged pool for {args.warmup} warm-up and {args.steps} timed cycles "
                 f"needs {pool_bytes / 2**30:.0f} GiB (every cycle's entries stay in the cache) "
                 f"and {free_bytes / 2**30:.0f} GiB are free; use fewer --steps")
    pool = torch.empty((kv.L, 2, kv.num_blocks, kv.block_size, kv.H, kv.D), dtype=torch.bfloat16, device=d)
    if kv.blocks:
        ids = sorted(kv.blocks)
        pool[:, :, torch.tensor(ids, device=d)] = bf(np.stack([kv.blocks[X][0] for X in ids], axis=2))
    cache = binding.PagedKVCache(pool, t(kv.block_tables), t(kv.seq_lens), t(kv.refcount),
                                 t(kv.free_list), torch.tensor([kv.free_count], dtype=torch.int32, device=d),
                                 torch.zeros(1, dtype=torch.int32, device=d))
    k_new, v_new, cu_new = bf(kv.k_new), bf(kv.v_new), t(kv.cu_new)
    B, K, V = vin.B, vin.K, vin.V
    out = torch.empty(K + B, dtype=torch.int32, device=d)
    nacc = torch.empty(B, dtype=torch.int32, device=d)
    nemit = torch.empty(B, dtype=torch.int32, device=d)
    err = torch.zeros(1, dtype=torch.int32, device=d)
    dt = binding.SPECDEC_BF16 if vin.dtype == "bf16" else binding.SPECDEC_F32
    pr = {}
    if args.per_request:
        pr["temperatures"] = torch.full((B,), vin.T, dtype=torch.float32, device=d)
        if 0 < vin.top_k < V:
            pr["top_ks"] = torch.full((B,), vin.top_k, dtype=torch.int32, device=d)
            pr["top_k_max"] = vin.top_k
        if 0.0 < top_p < 1.0:
            pr["top_ps"] = torch.full((B,), top_p, dtype=torch.float32, device=d)
    prm = binding._params(B, d, pr.get("temperatures"), pr.get("top_ks"), pr.get("top_ps"),
                          pr.get("top_k_max"))
    ws = torch.empty(binding.specdec_verify_workspace_size(B, K, V, dt, vin.top_k, top_p, prm),
                     dtype=torch.uint8, device=d)
    cws = torch.empty(binding.specdec_cycle_workspace_size(B, K, V, dt, vin.top_k, top_p, prm),
                      dtype=torch.uint8, device=d)
    kws = torch.empty(binding.kv_paged_append_workspace_size(B, K + B), dtype=torch.uint8, device=d)
    n = args.warmup + args.steps
    timed = [i for i in range(args.warmup, n) if (i - args.warmup) % max(args.timing_every, 1) == 0]
    evs = {i: (binding.HipEvent(), binding.HipEvent()) for i in timed}
    main_s = torch.cuda.current_stream(d)
    side_s = torch.cuda.Stream(d)                      # default priority
    ev_stats = [binding.HipEvent(timing=False) for _ in range(n + 2 * args.steps)]
    ev_kv = [binding.HipEvent(timing=False) for _ in range(n + 2 * args.steps)]

    # serial schedule: events around each call on the timing steps
    call_ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in timed}

    def step(i):
        dbg = binding.SpecdecDebug()
        if i in evs:
            dbg.ev_stats_begin, dbg.ev_stats_end = evs[i][0].handle, evs[i][1].handle
        ce = call_ev.get(i) if args.schedule == "serial" else None
        if args.schedule in ("fused", "early-exit"):
            binding.specdec_cycle(cache, k_new, v_new, tgt, dft, tokens, cu, u_acc, u_smp,
                                  max_k=vin.max_k, temperature=vin.T, top_k=vin.top_k,
                                  out_tokens=out, num_accepted=nacc, num_emitted=nemit,
                                  err_word=err, workspace=cws, debug=dbg, top_p=top_p,
                                  early_exit=args.schedule == "early-exit", **pr)
            return
        if args.schedule == "serial":
            if ce:
                ce[0].record()
            binding.kv_paged_append(cache, k_new, v_new, cu_new, kws)
            if ce:
                ce[1].record()
            binding.specdec_verify(tgt, dft, tokens, cu, u_acc, u_smp, max_k=vin.max_k,
                                   temperature=vin.T, top_k=vin.top_k, out_tokens=out,
                                   num_accepted=nacc, num_emitted=nemit, err_word=err,
                                   workspace=ws, debug=dbg, top_p=top_p, **pr)
            if ce:
                ce[2].record()
        else:
            dbg.ev_stats_done = ev_stats[i].handle
            binding.specdec_verify(tgt, dft, tokens, cu, u_acc, u_smp, max_k=vin.max_k,
                                   temperature=vin.T, top_k=vin.top_k, out_tokens=out,
                                   num_accepted=nacc, num_emitted=nemit, err_word=err,
                                   workspace=ws, debug=dbg, top_p=top_p, **pr)
            ev_stats[i].wait_on(side_s)
            with torch.cuda.stream(side_s):
                binding.kv_paged_append(cache, k_new, v_new, cu_new, kws)
            ev_kv[i].record(side_s)
            ev_kv[i].wait_on(main_s)
        binding.kv_rollback(cache, nacc, cu)
        if ce:
            ce[3].record()

    if args.calibrate_copy_mib:
        nb = args.calibrate_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=d).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.settle_ms > 0:
        # clocks rise over tens of milliseconds of load; the cycles run here leave no trace
        # in the cache state (its metadata is restored after every 16)
        c = cache
        meta = (c.block_tables, c.seq_lens, c.refcount, c.free_list, c.free_count, c.state)
        snap = [x.clone() for x in meta]
        err0 = err.clone()
        ts = time.perf_counter()
        while (time.perf_counter() - ts) * 1e3 < args.settle_ms:
            for _ in range(16):
                step(-1)
            for dst, src in zip(meta, snap):
                dst.copy_(src)
            torch.cuda.synchronize()
        err.copy_(err0)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, n):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = int(cache.state.item())
    if st:
        print(f"# warning: cache state word {st:#x}", file=sys.stderr)
    if int(err.item()) & (binding.ERR_TOKEN | binding.ERR_K | binding.ERR_NONFINITE | binding.ERR_UNIFORM):
        print(f"# warning: verify error word {int(err.item()):#x}", file=sys.stderr)
    stats_ms = [evs[i][0].elapsed_ms(evs[i][1]) for i in timed]
    stats_avg_s = float(np.mean(stats_ms)) / 1e3
    ms_per_step = elapsed / args.steps * 1e3
    # per-cycle times (median, p10, p90) from events around each of as many further cycles,
    # outside the timed region
    cyc = []
    for i in range(n, n + args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(i)
        e1.record()
        cyc.append((e0, e1))
    torch.cuda.synchronize()
    cyc_ms = np.array([a.elapsed_time(b) for a, b in cyc])
    # and as many again, each after a write of --flush-mib MiB outside its events
    cyc_fl_ms = None
    if args.flush_mib:
        junk = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=d)
        cyc = []
        for i in range(n + args.steps, n + 2 * args.steps):
            junk.fill_(i & 0xff)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(i)
            e1.record()
            cyc.append((e0, e1))
        torch.cuda.synchronize()
        cyc_fl_ms = np.array([a.elapsed_time(b) for a, b in cyc])
        del junk
    early_cmp = None
    if compare_early:
        # specdec_cycle_early_exit on the same batch: 10 untimed cycles, then as many as
        # the timed region, by wall clock
        def ee_step():
            binding.specdec_cycle(cache, k_new, v_new, tgt, dft, tokens, cu, u_acc, u_smp,
                                  max_k=vin.max_k, temperature=vin.T, top_k=vin.top_k,
                                  out_tokens=out, num_accepted=nacc, num_emitted=nemit,
                                  err_word=err, workspace=cws, top_p=top_p, early_exit=True,
                                  **pr)
        for _ in range(10):
            ee_step()
        torch.cuda.synchronize()
        te0 = time.perf_counter()
        for _ in range(args.steps):
            ee_step()
        torch.cuda.synchronize()
        ee_ms = (time.perf_counter() - te0) / args.steps * 1e3
        early_cmp = {"ms_per_step": ee_ms, "value": vin.K / (ee_ms / 1e3), "unit": "positions/s"}
    graph = None
    if args.graph and args.schedule in ("fused", "early-exit"):
        # one cycle captured (its launches read every size and pointer from device memory or
        # their arguments, so each replay is the next cycle), then replays timed like the
        # eager cycles
        gs = torch.cuda.Stream(d)
        gs.wait_stream(main_s)
        with torch.cuda.stream(gs):
            step(n + 2 * args.steps)                      # an eager cycle on the capture stream
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            step(n + 2 * args.steps + 1)
        torch.cuda.synchronize()
        for _ in range(min(args.warmup, args.steps)):
            g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - tg0) / args.steps * 1e3
        ev = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        g_cyc = np.array([a.elapsed_time(b) for a, b in ev])
        graph = {"ms_per_step": g_ms, "value": K / (g_ms / 1e3),
                 "cycle_ms_p10_p50_p90": [float(np.percentile(g_cyc, q)) for q in (10, 50, 90)]}
        del g
    acceptance = acceptance_stats(binding, torch, d, vin, tgt, dft, tokens, cu, u_acc, u_smp,
                                  out, nacc, nemit, err, ws, top_p, pr, ms_per_step)
    ceilings = None if args.no_ceilings else probe_ceilings(binding, torch, d, [tgt, dft], 512)
    es = 2 if vin.dtype == "bf16" else 4
    rows = 2 * K + B
    logit_bytes = rows * V * es
    kv_bytes = 2 * (K + B) * kv.L * 2 * kv.H * kv.D * 2      # read + write, K and V
    small = 4 * (3 * K + 6 * B + 2)                         # tokens, uniforms, offsets, outputs
    # the rows this batch's outputs depend on: each request's target and draft rows up to
    # its first rejection (its correction row included), or every row when all proposals
    # were accepted (the bonus row included); the full cycle reads the rest as well (every
    # proposal gets its statistics) but they decide nothing, and the early-exit cycle reads
    # exactly these
    kb = np.diff(np.asarray(vin.cu_draft, dtype=np.int64))
    ab = np.maximum(nacc.cpu().numpy().astype(np.int64), 0)
    seq_rows = int(np.where(ab < kb, 2 * (ab + 1), 2 * kb + 1).sum())
    ee_rows = early_exit_rows(kb, ab, binding.EARLY_EXIT_SEQUENTIAL)
    early = args.schedule == "early-exit"
    read_bytes = (ee_rows if early else rows) * V * es
    cycle_bytes = read_bytes + kv_bytes + small
    positions_per_s = K * args.steps / elapsed
    cycle_gbps = cycle_bytes / (ms_per_step / 1e3) / 1e9
    achieved = read_bytes / stats_avg_s / 1e9
    filtered = 0 < vin.top_k < V or 0.0 < top_p < 1.0
    # top_k above 1024 runs the multi-pass select inside the merge launch: no launch
    # streams the rows once
    generic = 0 < vin.top_k < V and vin.top_k > 1024
    # per-request arrays hold temperatures only when no top-k / top-p is on: plain statistics
    if early:                          # the position launches, timed as one span
        stats_kernel = "k_cycle_fpass" if filtered else "k_cycle_pass"
    elif filtered:                     # the chunk launch streams the rows
        # top-p alone (scalar) has a launch of its own in the fused cycle
        topp_alone = not args.per_request and not 0 < vin.top_k < V
        stats_kernel = (("k_cycle_topp" if topp_alone else "k_cycle_topk")
                        if args.schedule == "fused" else "k_topk_chunks")
    else:
        stats_kernel = (("k_cycle_stats_pr" if args.per_request else "k_cycle_stats")
                        if args.schedule == "fused" else "k_row_stats")
    res = {
        "metric": METRIC,
        "value": positions_per_s,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": vin.dtype,
        "data": "synthetic",
        "config": {"workload": (f"{wl.name}: B={B} k={'U{%d..%d}' % wl.k_range if wl.k_range else wl.k} "
                                f"V={V} {vin.dtype} T={vin.T:g} top_k={vin.top_k}"
                                + (f" top_p={top_p:g}" if 0.0 < top_p < 1.0 else "")
                                + (" (per-request arrays)" if args.per_request else "") + "; paged KV "
                                f"{kv.L}x{kv.H}x{kv.D} bf16, block {kv.block_size}"),
                   "global_batch": B, "positions_per_step": K, "parallelism": "single GPU",
                   "schedule": args.schedule},
        "cycle_ms_p10_p50_p90": [float(np.percentile(cyc_ms, q)) for q in (10, 50, 90)],
        "cycle_ms_p10_p50_p90_flushed": (None if cyc_fl_ms is None else
                                         [float(np.percentile(cyc_fl_ms, q)) for q in (10, 50, 90)]),
        "achieved_hbm_gbps": cycle_gbps,
        "pct_peak_hbm": 100.0 * cycle_gbps / PEAK_GBPS,
        "cycle_bytes": cycle_bytes,
        "roofline": {"bound": "hbm", "kernel": stats_kernel, "achieved": achieved,
                     "peak": PEAK_GBPS, "unit": "GB/s", "frac": achieved / PEAK_GBPS,
                     "traffic": None if early else traffic_from_profile(stats_kernel, wl.name),
                     "algorithmic_bytes": read_bytes,
                     "avg_launch_us": stats_avg_s * 1e6},
    }
    if early:
        # the events bracket every position launch (with top-k / top-p, their merge
        # launches too), and those launches also carry shares of the K/V scatter whose
        # bytes are not counted here: a span, not one launch at its roofline
        res["roofline"]["span"] = ("every statistics launch of the early-exit schedule, "
                                   "merges and K/V scatter shares included; "
                                   "algorithmic_bytes counts the logit rows read only")
    if args.schedule == "serial":
        # each call's time from events around it on the timing steps, and the bytes it must
        # move: the append reads and writes the new K/V, the verify reads every logit row
        # once, the rollback touches metadata only
        cms = lambda a_, b_: float(np.mean([call_ev[i][a_].elapsed_time(call_ev[i][b_]) for i in timed]))
        ap, ve, rb = cms(0, 1), cms(1, 2), cms(2, 3)
        res["per_call"] = {"append_ms": ap, "append_gbps": kv_bytes / (ap / 1e3) / 1e9,
                           "verify_ms": ve, "verify_gbps": logit_bytes / (ve / 1e3) / 1e9,
                           "rollback_ms": rb}
    if ceilings is not None:
        # the cycle's compulsory bytes at this device's measured ceilings: every logit row
        # read at the read probe's rate, the new K/V read and written at the copy probe's
        at = read_bytes / (ceilings["read_gbps"] * 1e9) + kv_bytes / (ceilings["copy_gbps"] * 1e9)
        ceilings["compulsory_ms_at_ceilings"] = at * 1e3
        ceilings["pct_peak_hbm_at_ceilings"] = 100.0 * cycle_bytes / at / 1e9 / PEAK_GBPS
        ceilings["cycle_vs_ceilings"] = at * 1e3 / ms_per_step
        res["ceilings"] = ceilings
        res["roofline"]["frac_of_read_ceiling"] = achieved / ceilings["read_gbps"]
    if generic:
        res["roofline"] = None
    seq_bytes = seq_rows * V * es + kv_bytes + small
    res["sequential_minimum"] = {"logit_rows": seq_rows, "logit_rows_streamed": rows,
                                 "cycle_bytes": seq_bytes,
                                 "gbps_at_measured_cycle": seq_bytes / (ms_per_step / 1e3) / 1e9}
    try:
        res["device_memory"] = binding.device_memory(d.index or 0)
    except Exception as e:   # reported, not needed for the line
        res["device_memory"] = {"error": str(e)}
    if graph is not None:
        res["graph"] = graph
    res["acceptance"] = acceptance
    if early_cmp is not None:
        # not the headline: the metric counts every logit row, which this cycle skips
        early_cmp["logit_rows_read"] = ee_rows
        early_cmp["cycle_bytes"] = ee_rows * V * es + kv_bytes + small
        early_cmp["achieved_hbm_gbps"] = early_cmp["cycle_bytes"] / (early_cmp["ms_per_step"] / 1e3) / 1e9
        early_cmp["logit_rows"] = rows
        res["early_exit"] = early_cmp
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(vin, kv, args.cpu_seconds, top_p)
        workers = args.cpu_workers or min(16, len(os.sched_getaffinity(0)))
        if workers > 1 and not args.per_request:
            res["cpu_baseline_ncores"] = cpu_baseline_ncores(vin, top_p, workers)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
