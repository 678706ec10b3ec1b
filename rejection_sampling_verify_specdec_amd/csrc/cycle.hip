// One whole speculative cycle in four launches (five with top-k or top-p; one more above
// 512 requests) (gfx950): the same work and results as kv_paged_append -> specdec_verify ->
// kv_rollback on one stream, with the latency-bound pieces folded into launches that are
// busy streaming memory anyway.
//
//   k_cycle_stats   workgroup 0 allocates the cycle's blocks (copy-on-write, LIFO pops,
//                   destination rows) while every other workgroup streams logit rows
//                   (row statistics; with top-k or top-p, k_cycle_topk gathers chunk
//                   candidates, k_cycle_topp for top-p alone, and a short per-row merge
//                   launch follows);
//   k_cycle_decide  one workgroup per request for its accept / reject decisions, then
//                   most of the K/V scatter;
//   k_cycle_part    workgroup 0 truncates every request to its committed prefix (up to 512
//                   requests; beyond that k_cycle_rollback runs after the pick) while the
//                   others sum the sampling weights chunk by chunk, then a share of the
//                   scatter;
//   k_cycle_pick    one workgroup per request draws its replacement / bonus token, then the
//                   rest of the scatter.
// The scatter (bandwidth-bound, independent of the decisions: every candidate is appended)
// is spread over the three launches after the statistics so that its copy fills the
// memory time the latency-bound decision, chunk-sum and pick workgroups leave idle. The
// early-exit cycle spreads it over its position launches instead.
//
// The cycle is the one the pages describe ("Walk through KV-cache updates when
// speculative decoding rejects some draft tokens": K/V for the candidates are appended by
// the verifying pass, the accept test runs left to right, pages past the committed prefix
// are freed): the pending token and the k_b proposals are appended (n_b = k_b + 1, new
// entry t of request b is row cu_draft[b] + b + t of k_new / v_new), then verified, then
// rolled back to the pending token plus the accepted proposals.

#include <algorithm>
#include <atomic>
#include <mutex>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "kv_dev.h"
#include "verify_dev.h"


namespace sd {

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kPartNT) void k_accept_part(SampleArgs a) {
    accept_part_body<BF16, VEC, kPartNT>(a, blockIdx.x / a.nch, blockIdx.x % a.nch);
}

template <bool BF16>
__global__ __launch_bounds__(kWave) void k_accept_final(SampleArgs a) {
    accept_final_body<BF16>(a, blockIdx.x);
}

constexpr int kCycAllocNT = kNT;   // allocation workgroup inside the statistics launch
constexpr int kCycScatterPPT = kScPPT;   // token rows per scatter thread in flight

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_cycle_stats(KvArgs kv, const int* __restrict__ cu,
                                                     int B, int N, uint8_t* __restrict__ aws,
                                                     const uint8_t* __restrict__ tgt,
                                                     const uint8_t* __restrict__ dft,
                                                     int rows_t, int V, int nchunks, float c,
                                                     RowPartial* __restrict__ part,
                                                     const RowParams* __restrict__ rpar) {
    if (blockIdx.x == 0) {
        alloc_body<kCycAllocNT>(kv, cu, 1, B, N, aws);
        return;
    }
    row_stats_body<BF16, VEC>(tgt, dft, rows_t, V, nchunks, c, part, blockIdx.x - 1, rpar);
}

// Per-request temperatures alone: the same launch, each workgroup deriving its row's
// parameters from its request's values (the first chunk's workgroup also records them for
// the launches that follow), so no parameter launch runs first.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_cycle_stats_pr(KvArgs kv, const int* __restrict__ cu,
                                                        int B, int N, uint8_t* __restrict__ aws,
                                                        const uint8_t* __restrict__ tgt,
                                                        const uint8_t* __restrict__ dft,
                                                        int rows_t, int V, int nchunks,
                                                        RowPartial* __restrict__ part,
                                                        ParamArgs pa) {
    __shared__ float s_c;
    if (blockIdx.x == 0) {
        alloc_body<kCycAllocNT>(kv, cu, 1, B, N, aws);
        return;
    }
    const int bid = blockIdx.x - 1, row = bid / nchunks;
    if (threadIdx.x == 0) {
        const RowParams rp = row_params_of(pa, row);
        if (bid == row * nchunks) pa.out[row] = rp;
        s_c = rp.c;
    }
    __syncthreads();
    row_stats_body<BF16, VEC>(tgt, dft, rows_t, V, nchunks, s_c, part, bid,
                              (const RowParams*)nullptr);
}

// One launch's share of the K/V scatter: scatter workgroups s0 .. s0 + ns - 1 of the
// ntiles * L * 2 (tile, layer / K-V plane) workgroups; each copies its tile's rows, and the
// copy-on-write copies are spread over all of them by global index.
struct ScatterShare {
    KvArgs kv;
    const uint8_t* knew;
    const uint8_t* vnew;
    const uint8_t* aws;
    int B, N, tpw, ntiles, s0, ns;
};

SD_DEV void scatter_share(const ScatterShare& sc, int i) {
    const int planes = sc.kv.L * 2;
    const int s = sc.s0 + i;
    scatter_body<kCycScatterPPT>(sc.kv, sc.knew, sc.vnew, sc.B, sc.N, sc.tpw, sc.aws, s / planes,
                                 s % planes, s, sc.ntiles * planes, kScNT);
}

// Of the n workgroups i = 0 .. n-1 of a launch, the last ns run the scatter: returns i's
// scatter index, or -1 with *work set to i (the launch's own work first in dispatch order).
SD_DEV int scatter_index(unsigned i, unsigned n, unsigned ns, int* work) {
    if (i >= n - ns) return (int)(i - (n - ns));
    *work = (int)i;
    return -1;
}

// Early-exit statistics: launch p holds the statistics of position p's rows (workgroup 0
// of launch 0 allocates the cycle's blocks first, as k_cycle_stats does); the launches
// after the first also carry a share of the K/V scatter (the allocation is done by then).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_cycle_pass(KvArgs kv, const int* __restrict__ cu,
                                                    int B, int N, uint8_t* __restrict__ aws,
                                                    SampleArgs sa, RowPartial* __restrict__ part,
                                                    int p, int nwg, ScatterShare sc) {
    if (p == 0) {
        if (blockIdx.x == 0) {
            alloc_body<kCycAllocNT>(kv, cu, 1, B, N, aws);
            return;
        }
        pass_body<BF16, VEC>(sa, part, 0, blockIdx.x - 1);
    } else {
        int w = 0;
        const int si = scatter_index(blockIdx.x, gridDim.x, sc.ns, &w);
        if (si >= 0) scatter_share(sc, si);
        else pass_body<BF16, VEC>(sa, part, p, w);
    }
}

// The early-exit cycle's last statistics launch (position p, every later row of each live
// request), with a share of the K/V scatter.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_cycle_tail(SampleArgs sa, RowPartial* __restrict__ part,
                                                    int p, int nwg, ScatterShare sc) {
    if (blockIdx.x < (unsigned)nwg) tail_body<BF16, VEC>(sa, part, p, blockIdx.x);
    else scatter_share(sc, blockIdx.x - nwg);
}

static_assert(kTkNT == kCycAllocNT, "allocation and top-k chunk workgroups share one launch");

// Early exit with a top-k / top-p transform: launch p runs the chunk select of position p's
// rows of the live requests (workgroup 0 of launch 0 allocates the cycle's blocks first;
// later launches carry a share of the K/V scatter); the tail launch every later row of the
// requests still live; a merge launch follows each (P2: 0 top-k, 1 top-p alone, 2
// per-request parameters).
template <bool BF16, bool VEC, int P2>
__global__ __launch_bounds__(kTkNT) void k_cycle_fpass(KvArgs kv, const int* __restrict__ cu,
                                                     int B, int N, uint8_t* __restrict__ aws,
                                                     SampleArgs sa, TopkArgs ta, int p,
                                                     ScatterShare sc) {
    if (p == 0) {
        if (blockIdx.x == 0) {
            alloc_body<kCycAllocNT>(kv, cu, 1, B, N, aws);
            return;
        }
        fpass_body<BF16, VEC, P2>(sa, ta, 0, blockIdx.x - 1);
    } else {
        int w = 0;
        const int si = scatter_index(blockIdx.x, gridDim.x, sc.ns, &w);
        if (si >= 0) scatter_share(sc, si);
        else fpass_body<BF16, VEC, P2>(sa, ta, p, w);
    }
}

template <bool BF16, bool VEC, int P2>
__global__ __launch_bounds__(kTkNT) void k_cycle_ftail(SampleArgs sa, TopkArgs ta, int p,
                                                     int nwg, ScatterShare sc) {
    if (blockIdx.x < (unsigned)nwg) ftail_body<BF16, VEC, P2>(sa, ta, p, blockIdx.x);
    else scatter_share(sc, blockIdx.x - nwg);
}

template <bool BF16, bool PR>
__global__ __launch_bounds__(kMergeNT) __attribute__((amdgpu_waves_per_eu(5))) void
k_cycle_fmerge(SampleArgs sa, TopkArgs ta, int p, int tail) {
    fmerge_body<BF16, kMergeNT, PR>(sa, ta, p, blockIdx.x, tail != 0);
}

// P2: 0 top-k, 1 top-p alone, 2 per-request parameters
template <bool BF16, bool VEC, int P2>
__global__ __launch_bounds__(kTkNT) void k_cycle_topk(KvArgs kv, const int* __restrict__ cu,
                                                      int B, int N, uint8_t* __restrict__ aws,
                                                      TopkArgs a) {
    if (blockIdx.x == 0) {
        alloc_body<kCycAllocNT>(kv, cu, 1, B, N, aws);
        return;
    }
    const int w = blockIdx.x - 1;
    if constexpr (P2 == 2) chunk_pr_body<BF16, VEC>(a, w / a.nchunks, w % a.nchunks);
    else topk_chunk_body<BF16, VEC, P2>(a, w / a.nchunks, w % a.nchunks,
                                        ChunkSel{a.top_k, a.c, P2 == 1});
}

// Top-p alone over 16-byte loads: the same launch held to 64 VGPRs, so that eight waves
// share each SIMD (the launch issues more instructions per byte than any other and hides
// its loads with waves; the scalar-load form would spill at this bound)
template <bool BF16>
__global__ __launch_bounds__(kTkNT) __attribute__((amdgpu_waves_per_eu(8))) void
k_cycle_topp(KvArgs kv, const int* __restrict__ cu, int B, int N, uint8_t* __restrict__ aws,
             TopkArgs a) {
    if (blockIdx.x == 0) {
        alloc_body<kCycAllocNT>(kv, cu, 1, B, N, aws);
        return;
    }
    const int w = blockIdx.x - 1;
    topk_chunk_body<BF16, true, 1>(a, w / a.nchunks, w % a.nchunks,
                                   ChunkSel{a.top_k, a.c, true});
}

template <bool BF16, bool PR, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(5))) void k_cycle_topk_merge(TopkArgs a) {
    if constexpr (PR) merge_pr_body<BF16, NT>(a, blockIdx.x);
    else topk_merge_body<BF16, NT>(a, blockIdx.x, RowSel{a.top_k, a.topp_mode, a.top_p, a.c});
}

__global__ __launch_bounds__(256) void k_cycle_row_params(ParamArgs a, int rows) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r < rows) row_params_one(a, r);
}

static_assert(kDecideNT == kScNT && kPartNT == kScNT && kPickNT == kScNT && kNT == kScNT,
              "scatter workgroups share the decision, chunk-sum, pick and position launches");

template <bool BF16>
__global__ __launch_bounds__(kDecideNT) void k_cycle_decide(SampleArgs sa, ScatterShare sc) {
    // the decision workgroups first: the launch that follows waits for them, not for the
    // scatter's tail
    const int bid = blockIdx.x;
    if (bid < sa.B) {
        decide_kernel_body<BF16, kDecideNT>(sa, bid);
        return;
    }
    scatter_share(sc, bid - sa.B);
}

// Up to kCycRbMaxB requests the rollback runs as workgroup 0 of the chunk-sum launch (its
// LDS then stays small), otherwise as a launch of its own after the draws.
constexpr int kCycRbMaxB = 512;
constexpr int kCycRbEv = 512;

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kPartNT) void k_cycle_part(SampleArgs sa, KvArgs kv, int rb,
                                                        ScatterShare sc) {
    if (rb && blockIdx.x == 0) {
        rollback_body<kPartNT, kCycRbMaxB, kCycRbEv>(kv, sa.num_acc, sa.cu, sa.B);
        return;
    }
    int w = 0;
    const int si = scatter_index(blockIdx.x - rb, gridDim.x - rb, sc.ns, &w);
    if (si >= 0) {
        scatter_share(sc, si);
        return;
    }
    part_body<BF16, VEC, kPartNT>(sa, w / sa.nch, w % sa.nch);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kPickNT) void k_cycle_pick(SampleArgs sa, ScatterShare sc) {
    int w = 0;
    const int si = scatter_index(blockIdx.x, gridDim.x, sc.ns, &w);
    if (si >= 0) {
        scatter_share(sc, si);
        return;
    }
    pick_body<BF16, VEC, kPickNT>(sa, w);
}

__global__ __launch_bounds__(kKvNT) void k_cycle_rollback(SampleArgs sa, KvArgs kv) {
    rollback_body(kv, sa.num_acc, sa.cu, sa.B);
}

// How a cycle spreads the K/V scatter (percent of its workgroups) over the launches that
// follow the allocation. The fused cycle puts most of it beside the decisions, and without
// top-k / top-p a fifth beside the chunk sums and the picks (measured: -0.9% at the
// headline workload; with top-k the merges' rows change the balance and the split costs
// 1-2%); the early-exit cycle, whose statistics launches past position 0 hold few rows,
// spreads it over them and the sampling launches.
struct ScatterSplit {
    int pass_pct;      // beside position 1's statistics (early exit)
    int tail_pct;      // beside the last statistics launch (early exit)
    int part_pct;      // beside the chunk sums
    int pick_pct;      // beside the picks; the rest beside the decisions
};
constexpr ScatterSplit kFusedSplit = {0, 0, 15, 5};
constexpr ScatterSplit kFusedFilteredSplit = {0, 0, 0, 0};
constexpr ScatterSplit kEarlySplit = {30, 30, 10, 10};

static int pct_of(int n, int pct) { return (int)(((long long)n * pct) / 100); }

static ScatterShare scatter_plan(const KvArgs& kv, const uint8_t* knew, const uint8_t* vnew,
                                 const uint8_t* aws, int B, int N) {
    ScatterShare sc;
    sc.kv = kv;
    sc.knew = knew;
    sc.vnew = vnew;
    sc.aws = aws;
    sc.B = B;
    sc.N = N;
    sc.tpw = scatter_tokens_per_wg(kv, kScNT, kCycScatterPPT);
    sc.ntiles = (N + sc.tpw - 1) / sc.tpw;
    sc.s0 = 0;
    sc.ns = sc.ntiles * kv.L * 2;
    return sc;
}

// sc's workgroups [from, from + n)
static ScatterShare scatter_slice(ScatterShare sc, int from, int n) {
    sc.s0 = from;
    sc.ns = n;
    return sc;
}

// decision, draw, rollback, with the scatter workgroups `sc` holds (whatever the position
// launches left) spread over them; analytics when asked
template <bool BF16, bool VEC>
static void launch_cycle_tail(const KvArgs& kv, int B, int K, const WsPlan& p,
                              const SampleArgs& sa, const ScatterShare& sc,
                              const ScatterSplit& split, hipStream_t st) {
    const int total = sc.s0 + sc.ns;          // the whole scatter; sc holds what is left
    const int n_pick = std::min(sc.ns, pct_of(total, split.pick_pct));
    const int n_part = std::min(sc.ns - n_pick, pct_of(total, split.part_pct));
    const int n_dec = sc.ns - n_pick - n_part;
    const ScatterShare s_dec = scatter_slice(sc, sc.s0, n_dec);
    const ScatterShare s_part = scatter_slice(sc, sc.s0 + n_dec, n_part);
    const ScatterShare s_pick = scatter_slice(sc, sc.s0 + n_dec + n_part, n_pick);
    hipLaunchKernelGGL((k_cycle_decide<BF16>), dim3((unsigned)B + (unsigned)n_dec), dim3(kDecideNT),
                       0, st, sa, s_dec);
    const int rb = B <= kCycRbMaxB;
    hipLaunchKernelGGL((k_cycle_part<BF16, VEC>), dim3((unsigned)B * p.nch + rb + (unsigned)n_part),
                       dim3(kPartNT), 0, st, sa, kv, rb, s_part);
    hipLaunchKernelGGL((k_cycle_pick<BF16, VEC>), dim3((unsigned)B + (unsigned)n_pick), dim3(kPickNT),
                       0, st, sa, s_pick);
    if (sa.prec && K > 0) {
        // acceptance analytics: residual mass of every proposal position, then beta and E[A]
        hipLaunchKernelGGL((k_accept_part<BF16, VEC>), dim3((unsigned)K * p.nch), dim3(kPartNT), 0,
                           st, sa);
        hipLaunchKernelGGL((k_accept_final<BF16>), dim3(B), dim3(kWave), 0, st, sa);
    } else if (sa.prec) {
        hipLaunchKernelGGL((k_accept_final<BF16>), dim3(B), dim3(kWave), 0, st, sa);
    }
    if (!rb) hipLaunchKernelGGL(k_cycle_rollback, dim3(1), dim3(kKvNT), 0, st, sa, kv);
}

template <bool BF16, bool VEC>
static void launch_cycle(const KvArgs& kv, const uint8_t* knew, const uint8_t* vnew,
                         const uint8_t* tgt, const uint8_t* dft, const int* cu, int B, int K,
                         int V, float top_p, float c, const WsPlan& p, uint8_t* vws, uint8_t* aws,
                         const SampleArgs& sa, const ParamArgs& pa, const specdec_debug* dbg,
                         hipStream_t st) {
    const int rows = 2 * K + B;
    const int N = K + B;
    RowPartial* part = reinterpret_cast<RowPartial*>(vws + p.part);
    hipEvent_t e0 = dbg ? dbg->ev_stats_begin : nullptr;
    hipEvent_t e1 = dbg ? dbg->ev_stats_end : nullptr;
    if (p.pr_plain) {
        hipExtLaunchKernelGGL((k_cycle_stats_pr<BF16, VEC>), dim3((unsigned)rows * p.nchunks + 1),
                              dim3(kNT), 0, st, e0, e1, 0, kv, cu, B, N, aws, tgt, dft, K + B, V,
                              p.nchunks, part, pa);
    } else if (p.pr) {
        const TopkArgs ta = topk_args(tgt, dft, K + B, V, top_p, c, p, vws);
        hipLaunchKernelGGL(k_cycle_row_params, dim3((unsigned)(rows + 255) / 256), dim3(256), 0, st,
                           pa, rows);
        hipExtLaunchKernelGGL((k_cycle_topk<BF16, VEC, 2>), dim3((unsigned)rows * p.nchunks + 1),
                              dim3(kTkNT), 0, st, e0, e1, 0, kv, cu, B, N, aws, ta);
        hipLaunchKernelGGL((k_cycle_topk_merge<BF16, true, kMergeNT>), dim3(rows),
                           dim3(kMergeNT), 0, st, ta);
    } else if (p.filter) {
        const TopkArgs ta = topk_args(tgt, dft, K + B, V, top_p, c, p, vws);
        const unsigned nchunk_wg = ta.generic ? 0u : (unsigned)rows * p.nchunks;
        if (p.topp_mode == 2 && VEC)
            hipExtLaunchKernelGGL((k_cycle_topp<BF16>), dim3(nchunk_wg + 1), dim3(kTkNT), 0, st,
                                  e0, e1, 0, kv, cu, B, N, aws, ta);
        else if (p.topp_mode == 2)
            hipExtLaunchKernelGGL((k_cycle_topk<BF16, VEC, 1>), dim3(nchunk_wg + 1), dim3(kTkNT),
                                  0, st, e0, e1, 0, kv, cu, B, N, aws, ta);
        else
            hipExtLaunchKernelGGL((k_cycle_topk<BF16, VEC, 0>), dim3(nchunk_wg + 1), dim3(kTkNT),
                                  0, st, e0, e1, 0, kv, cu, B, N, aws, ta);
        hipLaunchKernelGGL((k_cycle_topk_merge<BF16, false, kMergeNT>), dim3(rows),
                           dim3(kMergeNT), 0, st, ta);
    } else {
        hipExtLaunchKernelGGL((k_cycle_stats<BF16, VEC>), dim3((unsigned)rows * p.nchunks + 1),
                              dim3(kNT), 0, st, e0, e1, 0, kv, cu, B, N, aws, tgt, dft, K + B, V,
                              p.nchunks, c, part, (const RowParams*)nullptr);
    }
    if (dbg && dbg->ev_stats_done) (void)hipEventRecord(dbg->ev_stats_done, st);
    launch_cycle_tail<BF16, VEC>(kv, B, K, p, sa, scatter_plan(kv, knew, vnew, aws, B, N),
                                 p.filter ? kFusedFilteredSplit : kFusedSplit, st);
}

// The early-exit cycle: one statistics launch for each of positions 0 .. kEarlyCut - 1,
// then one for every later row of the requests still live, with the K/V scatter spread over
// the launches after the first; then the same decision, draw and cache launches. With a
// top-k / top-p transform each statistics launch is a chunk-select launch followed by a
// merge launch over the rows it selected.
template <bool BF16, bool VEC, int P2>
static void launch_cycle_early_filtered(const KvArgs& kv, const uint8_t* knew,
                                        const uint8_t* vnew, const int* cu, int B, int K,
                                        int max_k, const WsPlan& p, const TopkArgs& ta,
                                        const SampleArgs& sa, const ParamArgs& pa,
                                        uint8_t* aws, const specdec_debug* dbg, hipStream_t st) {
    constexpr bool PR = P2 == 2;
    if (PR) {                   // each row's parameters first
        const int rows = 2 * K + B;
        hipLaunchKernelGGL(k_cycle_row_params, dim3((unsigned)(rows + 255) / 256), dim3(256), 0, st,
                           pa, rows);
    }
    const unsigned nwg = (unsigned)B * 2u * (unsigned)ta.nchunks;
    const ScatterShare sc = scatter_plan(kv, knew, vnew, aws, B, K + B);
    if (dbg && dbg->ev_stats_begin) (void)hipEventRecord(dbg->ev_stats_begin, st);
    int done = 0;
    for (int q = 0; q <= max_k && q < kEarlyCut; ++q) {
        const int share = q == 1 ? std::min(sc.ns, pct_of(sc.ns, kEarlySplit.pass_pct)) : 0;
        hipLaunchKernelGGL((k_cycle_fpass<BF16, VEC, P2>),
                           dim3(nwg + (q == 0 ? 1u : 0u) + (unsigned)share), dim3(kTkNT), 0, st,
                           kv, cu, B, K + B, aws, sa, ta, q, scatter_slice(sc, done, share));
        done += share;
        hipLaunchKernelGGL((k_cycle_fmerge<BF16, PR>), dim3((unsigned)B * 2u), dim3(kMergeNT), 0,
                           st, sa, ta, q, 0);
    }
    if (max_k >= kEarlyCut) {
        const unsigned per = (unsigned)early_tail_slots(max_k, kEarlyCut);
        const unsigned tw = (unsigned)B * per * (unsigned)ta.nchunks;
        const int share = std::min(sc.ns - done, pct_of(sc.ns, kEarlySplit.tail_pct));
        hipLaunchKernelGGL((k_cycle_ftail<BF16, VEC, P2>), dim3(tw + (unsigned)share), dim3(kTkNT),
                           0, st, sa, ta, kEarlyCut, (int)tw, scatter_slice(sc, done, share));
        done += share;
        hipLaunchKernelGGL((k_cycle_fmerge<BF16, PR>), dim3((unsigned)B * per), dim3(kMergeNT), 0,
                           st, sa, ta, kEarlyCut, 1);
    }
    if (dbg && dbg->ev_stats_end) (void)hipEventRecord(dbg->ev_stats_end, st);
    if (dbg && dbg->ev_stats_done) (void)hipEventRecord(dbg->ev_stats_done, st);
    launch_cycle_tail<BF16, VEC>(kv, B, K, p, sa, scatter_slice(sc, done, sc.ns - done),
                                 kEarlySplit, st);
}

template <bool BF16, bool VEC>
static void launch_cycle_early(const KvArgs& kv, const uint8_t* knew, const uint8_t* vnew,
                               const uint8_t* tgt, const uint8_t* dft, const int* cu, int B,
                               int K, int max_k, int V, float top_p, float c, const WsPlan& p,
                               uint8_t* vws, uint8_t* aws, const SampleArgs& sa,
                               const ParamArgs& pa, const specdec_debug* dbg, hipStream_t st) {
    if (p.filter) {
        const TopkArgs ta = topk_args(tgt, dft, K + B, V, top_p, c, p, vws);
        if (p.pr)
            launch_cycle_early_filtered<BF16, VEC, 2>(kv, knew, vnew, cu, B, K, max_k, p, ta, sa,
                                                      pa, aws, dbg, st);
        else if (p.topp_mode == 2)
            launch_cycle_early_filtered<BF16, VEC, 1>(kv, knew, vnew, cu, B, K, max_k, p, ta, sa,
                                                      pa, aws, dbg, st);
        else
            launch_cycle_early_filtered<BF16, VEC, 0>(kv, knew, vnew, cu, B, K, max_k, p, ta, sa,
                                                      pa, aws, dbg, st);
        return;
    }
    RowPartial* part = reinterpret_cast<RowPartial*>(vws + p.part);
    if (p.pr_plain) {          // per-request temperatures: each row's log2(e) / T first
        const int rows = 2 * K + B;
        hipLaunchKernelGGL(k_cycle_row_params, dim3((unsigned)(rows + 255) / 256), dim3(256), 0, st,
                           pa, rows);
    }
    const unsigned nwg = (unsigned)B * 2u * (unsigned)p.nchunks;
    const ScatterShare sc = scatter_plan(kv, knew, vnew, aws, B, K + B);
    if (dbg && dbg->ev_stats_begin) (void)hipEventRecord(dbg->ev_stats_begin, st);
    int done = 0;
    for (int q = 0; q <= max_k && q < kEarlyCut; ++q) {
        const int share = q == 1 ? std::min(sc.ns, pct_of(sc.ns, kEarlySplit.pass_pct)) : 0;
        hipLaunchKernelGGL((k_cycle_pass<BF16, VEC>),
                           dim3(nwg + (q == 0 ? 1u : 0u) + (unsigned)share), dim3(kNT), 0, st, kv,
                           cu, B, K + B, aws, sa, part, q, (int)nwg,
                           scatter_slice(sc, done, share));
        done += share;
    }
    if (max_k >= kEarlyCut) {
        const unsigned tw = (unsigned)B * (unsigned)p.nchunks;
        const int share = std::min(sc.ns - done, pct_of(sc.ns, kEarlySplit.tail_pct));
        hipLaunchKernelGGL((k_cycle_tail<BF16, VEC>), dim3(tw + (unsigned)share), dim3(kNT), 0, st,
                           sa, part, kEarlyCut, (int)tw, scatter_slice(sc, done, share));
        done += share;
    }
    if (dbg && dbg->ev_stats_end) (void)hipEventRecord(dbg->ev_stats_end, st);
    if (dbg && dbg->ev_stats_done) (void)hipEventRecord(dbg->ev_stats_done, st);
    launch_cycle_tail<BF16, VEC>(kv, B, K, p, sa, scatter_slice(sc, done, sc.ns - done),
                                 kEarlySplit, st);
}

}  // namespace sd

extern "C" size_t specdec_cycle_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype,
                                               int32_t top_k, float top_p,
                                               const specdec_params* per_request) {
    if (B < 1 || K < 0 || V < 1 || V > SPECDEC_MAX_V || (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) ||
        (top_p != top_p && !(per_request && per_request->top_p)) ||
        (per_request && per_request->top_k && per_request->top_k_max < 0))
        return 0;
    return sd::align256(sd::plan_ws(B, K, V, dtype, top_k, top_p, per_request).total) +
           sd::append_ws_bytes(B, K + B);
}

static int cycle_entry(bool early, const kv_paged_cache* cache, const void* k_new,
                       const void* v_new, const void* target_logits, const void* draft_logits,
                       int32_t dtype, const int32_t* draft_tokens, const int32_t* cu_draft,
                       const float* u_accept, const float* u_sample, int32_t B, int32_t K,
                       int32_t max_k, int32_t V, float temperature, int32_t top_k, float top_p,
                       const specdec_params* per_request, int32_t* out_tokens,
                       int32_t* num_accepted, int32_t* num_emitted, int32_t* err_word,
                       const specdec_debug* dbg, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    using namespace sd;
    // early exit: no analytics (they need every row)
    if (early && dbg && (dbg->accept_prob || dbg->expected_emitted)) return SPECDEC_EINVAL;
    // verification arguments: the same checks as specdec_verify
    if (B < 1 || K < 0 || V < 1 || max_k < 0 || max_k > SPECDEC_MAX_K) return SPECDEC_EINVAL;
    if ((long long)K > (long long)B * max_k) return SPECDEC_EINVAL;
    if (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) return SPECDEC_EINVAL;
    const bool pr_t = per_request && per_request->temperature;
    const bool pr_p = per_request && per_request->top_p;
    if (!pr_t && (!(temperature > 0.0f) || !isfinite(temperature))) return SPECDEC_EINVAL;
    if (!pr_p && top_p != top_p) return SPECDEC_EINVAL;
    if (per_request && per_request->top_k && per_request->top_k_max < 0) return SPECDEC_EINVAL;
    if (!target_logits || !cu_draft || !u_sample || !out_tokens || !num_accepted ||
        !num_emitted || !err_word)
        return SPECDEC_EINVAL;
    if (K > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SPECDEC_EINVAL;
    // cache arguments: the same checks as kv_paged_append / kv_rollback
    if (!geometry_ok(cache) || B > SPECDEC_MAX_KV_BATCH || !k_new || !v_new ||
        ((uintptr_t)k_new & 15) || ((uintptr_t)v_new & 15))
        return SPECDEC_EINVAL;
    const WsPlan p = plan_ws(B, K, V, dtype, top_k, top_p, per_request);
    if ((size_t)(2 * (size_t)K + B) * p.nchunks + 1 > 0x7fffffffu ||
        (size_t)K * p.nch > 0x7fffffffu || V > SPECDEC_MAX_V ||
        (early && max_k >= kEarlyCut &&
         (size_t)B * early_tail_slots(max_k, kEarlyCut) * p.nchunks > 0x7fffffffu))
        return SPECDEC_EINVAL;
    const size_t vbytes = align256(p.total);
    if (!workspace || workspace_bytes < vbytes + append_ws_bytes(B, K + B) ||
        ((uintptr_t)workspace & 15))
        return SPECDEC_EWORKSPACE;

    const double c64 = 1.4426950408889634074 / (double)temperature;   // log2(e) / T
    const float c = pr_t ? 1.0f : (float)c64;
    if (!(c > 0.0f) || !isfinite(c)) return SPECDEC_EINVAL;
    const int es = dtype == SPECDEC_BF16 ? 2 : 4;
    const bool vec = ((size_t)V * es) % 16 == 0 && ((uintptr_t)target_logits & 15) == 0 &&
                     (K == 0 || ((uintptr_t)draft_logits & 15) == 0);
    uint8_t* vws = reinterpret_cast<uint8_t*>(workspace);
    uint8_t* aws = vws + vbytes;
    const uint8_t* tgt = reinterpret_cast<const uint8_t*>(target_logits);
    const uint8_t* dft = reinterpret_cast<const uint8_t*>(K > 0 ? draft_logits : target_logits);
    const uint8_t* knew = reinterpret_cast<const uint8_t*>(k_new);
    const uint8_t* vnew = reinterpret_cast<const uint8_t*>(v_new);

    SampleArgs sa;
    sa.tgt = tgt;
    sa.dft = dft;
    sa.tokens = draft_tokens;
    sa.cu = cu_draft;
    sa.u_acc = u_accept;
    sa.u_smp = u_sample;
    sa.B = B;
    sa.K = K;
    sa.max_k = max_k;
    sa.V = V;
    sa.nparts = p.nparts;
    sa.nch = p.nch;
    sa.topk = p.filter;
    sa.c = c;
    sa.T = temperature;
    sa.temps = pr_t ? per_request->temperature : nullptr;
    sa.eos = per_request ? per_request->eos_token : nullptr;
    sa.cap = per_request ? per_request->max_emit : nullptr;
    sa.early = early ? 1 : 0;
    sa.live = reinterpret_cast<int*>(vws + p.live);
    sa.rpar = p.pr ? reinterpret_cast<const RowParams*>(vws + p.rpar) : nullptr;
    sa.part = reinterpret_cast<const RowPartial*>(vws + p.part);
    sa.row_thr = reinterpret_cast<const float*>(vws + p.thr);
    sa.rec = reinterpret_cast<Decision*>(vws + p.rec);
    sa.wsum = reinterpret_cast<double*>(vws + p.wsum);
    sa.kn = p.tk_listed ? reinterpret_cast<const int*>(vws + p.tk_kn) : nullptr;
    sa.ktok = p.tk_listed ? reinterpret_cast<const uint32_t*>(vws + p.tk_ktok) : nullptr;
    sa.kkey = p.tk_listed ? reinterpret_cast<const uint16_t*>(vws + p.tk_kkey) : nullptr;
    sa.out_tokens = out_tokens;
    sa.num_acc = num_accepted;
    sa.num_emit = num_emitted;
    sa.err_word = err_word;
    sa.dbg = dbg ? *dbg : specdec_debug{};
    const bool analytics = dbg && (dbg->accept_prob || dbg->expected_emitted);
    sa.prec = analytics ? reinterpret_cast<Decision*>(vws + p.prec) : nullptr;
    sa.wacc = analytics ? reinterpret_cast<double*>(vws + p.wacc) : nullptr;

    const KvArgs kv = args_of(cache);
    ParamArgs pa{};
    if (p.pr) pa = param_args(cu_draft, B, K, V, temperature, top_k, top_p, per_request, p, vws);
    (void)hipGetLastError();
    if (early) {
        if (dtype == SPECDEC_BF16) {
            if (vec) launch_cycle_early<true, true>(kv, knew, vnew, tgt, dft, cu_draft, B, K, max_k, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
            else launch_cycle_early<true, false>(kv, knew, vnew, tgt, dft, cu_draft, B, K, max_k, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
        } else {
            if (vec) launch_cycle_early<false, true>(kv, knew, vnew, tgt, dft, cu_draft, B, K, max_k, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
            else launch_cycle_early<false, false>(kv, knew, vnew, tgt, dft, cu_draft, B, K, max_k, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
        }
    } else if (dtype == SPECDEC_BF16) {
        if (vec) launch_cycle<true, true>(kv, knew, vnew, tgt, dft, cu_draft, B, K, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
        else launch_cycle<true, false>(kv, knew, vnew, tgt, dft, cu_draft, B, K, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
    } else {
        if (vec) launch_cycle<false, true>(kv, knew, vnew, tgt, dft, cu_draft, B, K, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
        else launch_cycle<false, false>(kv, knew, vnew, tgt, dft, cu_draft, B, K, V, top_p, c, p, vws, aws, sa, pa, dbg, stream);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

extern "C" int specdec_cycle(const kv_paged_cache* cache, const void* k_new, const void* v_new,
                             const void* target_logits, const void* draft_logits, int32_t dtype,
                             const int32_t* draft_tokens, const int32_t* cu_draft,
                             const float* u_accept, const float* u_sample, int32_t B, int32_t K,
                             int32_t max_k, int32_t V, float temperature, int32_t top_k,
                             float top_p, const specdec_params* per_request, int32_t* out_tokens,
                             int32_t* num_accepted, int32_t* num_emitted, int32_t* err_word,
                             const specdec_debug* dbg, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    return cycle_entry(false, cache, k_new, v_new, target_logits, draft_logits, dtype,
                       draft_tokens, cu_draft, u_accept, u_sample, B, K, max_k, V, temperature,
                       top_k, top_p, per_request, out_tokens, num_accepted, num_emitted, err_word,
                       dbg, workspace, workspace_bytes, stream);
}

extern "C" int specdec_cycle_early_exit(const kv_paged_cache* cache, const void* k_new,
                                        const void* v_new, const void* target_logits,
                                        const void* draft_logits, int32_t dtype,
                                        const int32_t* draft_tokens, const int32_t* cu_draft,
                                        const float* u_accept, const float* u_sample, int32_t B,
                                        int32_t K, int32_t max_k, int32_t V, float temperature,
                                        int32_t top_k, float top_p,
                                        const specdec_params* per_request, int32_t* out_tokens,
                                        int32_t* num_accepted, int32_t* num_emitted,
                                        int32_t* err_word, const specdec_debug* dbg,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    return cycle_entry(true, cache, k_new, v_new, target_logits, draft_logits, dtype,
                       draft_tokens, cu_draft, u_accept, u_sample, B, K, max_k, V, temperature,
                       top_k, top_p, per_request, out_tokens, num_accepted, num_emitted, err_word,
                       dbg, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------------------
// specdec_cycle_static: the cycle over a scratch array in the device image instead of a
// caller workspace. The array's host-side name is only a stand-in for the symbol; the
// kernels get the device address that hipGetSymbolAddress returns, taken once per device
// (under a lock) with that device current, and kept.
// ---------------------------------------------------------------------------------------
namespace {

constexpr int kMaxScratchDevices = 64;
__device__ __align__(256) uint8_t scratch[SPECDEC_STATIC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_lock;

// the calling thread's current device's copy of the array, or null
void* scratch_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        p = q;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" int specdec_cycle_static(const kv_paged_cache* cache, const void* k_new,
                                    const void* v_new, const void* target_logits,
                                    const void* draft_logits, int32_t dtype,
                                    const int32_t* draft_tokens, const int32_t* cu_draft,
                                    const float* u_accept, const float* u_sample, int32_t B,
                                    int32_t K, int32_t max_k, int32_t V, float temperature,
                                    int32_t top_k, float top_p, const specdec_params* per_request,
                                    int32_t* out_tokens, int32_t* num_accepted,
                                    int32_t* num_emitted, int32_t* err_word,
                                    const specdec_debug* dbg, hipStream_t stream) {
    // the size check first: an oversized call never takes the array's address
    const size_t need = specdec_cycle_workspace_size(B, K, V, dtype, top_k, top_p, per_request);
    if (need > SPECDEC_STATIC_SCRATCH_BYTES) return SPECDEC_ESCRATCH;
    void* ws = scratch_of_current_device();
    if (!ws) return SPECDEC_EHIP;
    return cycle_entry(false, cache, k_new, v_new, target_logits, draft_logits, dtype,
                       draft_tokens, cu_draft, u_accept, u_sample, B, K, max_k, V, temperature,
                       top_k, top_p, per_request, out_tokens, num_accepted, num_emitted, err_word,
                       dbg, ws, SPECDEC_STATIC_SCRATCH_BYTES, stream);
}
