// Verification of draft trees for gfx950: a team of 1024-thread workgroups walks each
// request's tree, sharing every pass over a row (tree_dev.h). With top-k or top-p, the
// linear path's chunk select and merge first give every target and draft row its
// threshold and the max and exp-sum of its kept tokens, which the walk reads in place of
// its own statistics passes; a bf16 target row's kept tokens are also listed (up to
// kKeptCap), and the walk's passes and draw over such a row read the list alone. The cache step that keeps the accepted path is kv_tree_commit
// (kv.hip).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include "tree_dev.h"

namespace sd {

// Block x serves request x % Bp as member x / Bp (Bp: B rounded up to a multiple of 8):
// every request's first member is dispatched before any second one, and blocks are dealt
// to the 8 XCDs in turn, so the members of a team share an XCD (and its L2) when the
// dispatcher keeps that order; nothing depends on it.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kTreeNT) void k_tree_verify(TreeArgs a) {
    const int Bp = (a.B + 7) / 8 * 8;
    const int b = blockIdx.x % Bp, mem = blockIdx.x / Bp;
    if (b >= a.B) return;
    tree_walk_body<BF16, VEC>(a, b, mem);
}

// the team counters and (with top-k / top-p) the draft rows' marks start at zero
__global__ void k_tree_reset(int* ctr, int n, int* need, int nn) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) ctr[i] = 0;
    if (i < nn) need[i] = 0;
}

// With top-k / top-p only positions with children have their draft rows read: node i
// marks its parent's position (bounds-checked; a malformed tree fails in the walk).
__global__ void k_tree_mark(const int* __restrict__ cu, const int* __restrict__ parent, int B,
                            int N, int* __restrict__ need) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    int lo = 0, hi = B;                         // largest b with cu[b] <= i
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= i) lo = mid;
        else hi = mid;
    }
    const int j = i - cu[lo], pa = parent[i];
    const long long row = (long long)cu[lo] + lo + pa + 1;
    if (j >= 0 && pa >= -1 && pa < j && row >= 0 && row < (long long)N + B) need[row] = 1;
}

// a draft row no walk reads (the position of a leaf) is skipped
SD_DEV bool tree_row_skipped(const TopkArgs& a, const int* need, int row) {
    return row >= a.rows_t && need[row - a.rows_t] == 0;
}

// the select of every row (target rows first, then draft rows), as in the linear path
template <bool BF16, bool VEC, bool P2>
__global__ __launch_bounds__(kTkNT) void k_tree_select(TopkArgs a, const int* need) {
    const int row = blockIdx.x / a.nchunks;
    if (tree_row_skipped(a, need, row)) return;
    topk_chunk_body<BF16, VEC, P2 ? 1 : 0>(a, row, blockIdx.x % a.nchunks,
                                          ChunkSel{a.top_k, a.c, P2});
}

// top-p alone over 16-byte loads, held to 64 VGPRs (eight waves per SIMD)
template <bool BF16>
__global__ __launch_bounds__(kTkNT) __attribute__((amdgpu_waves_per_eu(8))) void
k_tree_topp(TopkArgs a, const int* need) {
    const int row = blockIdx.x / a.nchunks;
    if (tree_row_skipped(a, need, row)) return;
    topk_chunk_body<BF16, true, 1>(a, row, blockIdx.x % a.nchunks,
                                   ChunkSel{a.top_k, a.c, true});
}

template <bool BF16, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(5))) void k_tree_merge(TopkArgs a, const int* need) {
    if (tree_row_skipped(a, need, blockIdx.x)) return;
    topk_merge_body<BF16, NT>(a, blockIdx.x, RowSel{a.top_k, a.topp_mode, a.top_p, a.c});
}

// per-request transforms: each row's parameters, then its chunks and merge (the linear
// path's per-request bodies over the tree's rows)
__global__ __launch_bounds__(256) void k_tree_params(ParamArgs a, int rows) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r < rows) row_params_one(a, r);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kTkNT) void k_tree_select_pr(TopkArgs a, const int* need) {
    const int row = blockIdx.x / a.nchunks;
    if (tree_row_skipped(a, need, row)) return;
    chunk_pr_body<BF16, VEC>(a, row, blockIdx.x % a.nchunks);
}

template <bool BF16, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(5))) void k_tree_merge_pr(TopkArgs a, const int* need) {
    if (tree_row_skipped(a, need, blockIdx.x)) return;
    merge_pr_body<BF16, NT>(a, blockIdx.x);
}

struct TreeWs {
    size_t ctr_bytes, ring_bytes, total, need;
    int nchunk, nsub, slot;
    WsPlan sel;                         // top-k / top-p: offsets from the workspace start
};

static bool tree_ws(int32_t B, int32_t N, int32_t V, int32_t dtype, int32_t top_k, float top_p,
                    const specdec_params* prm, TreeWs* w) {
    if (B < 1 || N < 0 || V < 1 || V > SPECDEC_MAX_V) return false;
    if (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) return false;
    if (top_p != top_p && !(prm && prm->top_p)) return false;
    if (prm && (prm->eos_token || prm->max_emit)) return false;   // no stopping on trees
    if (prm && prm->top_k && prm->top_k_max < 0) return false;
    w->nchunk = (V + kTreeChunk - 1) / kTreeChunk;
    w->nsub = (V + kTreeSub - 1) / kTreeSub;
    w->slot = 64 * w->nchunk;           // >= 4 * nsub (weights); 4 per wave-chunk (stats)
    w->ctr_bytes = ((size_t)B * kTreeCtrStride * sizeof(int) + 255) & ~(size_t)255;
    w->ring_bytes = ((size_t)N + 2 * (size_t)B) * w->slot * sizeof(double);
    size_t off = align256(w->ctr_bytes + w->ring_bytes);
    w->sel = plan_transform(V, dtype, top_k, top_p, prm);
    const size_t rows = 2 * ((size_t)N + B);
    if (w->sel.pr) {
        w->sel.rpar = off;
        off = align256(off + rows * sizeof(RowParams));
    }
    w->need = off;
    if (w->sel.filter) {
        off = align256(off + ((size_t)N + B) * sizeof(int));     // draft rows read
        w->sel.part = off;
        off = align256(off + rows * sizeof(RowPartial));
        w->sel.thr = off;
        off = align256(off + rows * sizeof(float));
        off = plan_select(w->sel, off, rows, (size_t)N + B, dtype, true);
    }
    w->total = off;
    return true;
}

}  // namespace sd

extern "C" size_t specdec_tree_verify_workspace_size(int32_t B, int32_t N, int32_t V,
                                                     int32_t dtype, int32_t top_k, float top_p,
                                                     const specdec_params* per_request) {
    sd::TreeWs w;
    return sd::tree_ws(B, N, V, dtype, top_k, top_p, per_request, &w) ? w.total : 0;
}

extern "C" int specdec_tree_verify(const void* target_logits, const void* draft_logits,
                                   int32_t dtype, const int32_t* tree_tokens,
                                   const int32_t* tree_parent, const int32_t* cu_nodes,
                                   const float* u_accept, const float* u_sample, int32_t B,
                                   int32_t N, int32_t max_nodes, int32_t V, float temperature,
                                   int32_t top_k, float top_p, const specdec_params* per_request,
                                   int32_t* out_tokens, int32_t* accepted_nodes,
                                   int32_t* num_accepted, int32_t* num_emitted,
                                   int32_t* err_word, int32_t* req_flags, int32_t team,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    using namespace sd;
    if (B < 1 || N < 0 || V < 1 || V > SPECDEC_MAX_V || max_nodes < 0 ||
        max_nodes > SPECDEC_MAX_TREE)
        return SPECDEC_EINVAL;
    if ((long long)N > (long long)B * max_nodes) return SPECDEC_EINVAL;
    if (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) return SPECDEC_EINVAL;
    const bool pr_t = per_request && per_request->temperature;
    if (!pr_t && (!(temperature > 0.0f) || !isfinite(temperature))) return SPECDEC_EINVAL;
    if (top_p != top_p && !(per_request && per_request->top_p)) return SPECDEC_EINVAL;
    if (!target_logits || !draft_logits || !cu_nodes || !u_sample || !out_tokens ||
        !num_accepted || !num_emitted || !err_word)
        return SPECDEC_EINVAL;
    if (N > 0 && (!tree_tokens || !tree_parent || !u_accept || !accepted_nodes))
        return SPECDEC_EINVAL;
    // log2(e) / T (per-request temperatures: each row's own, from the parameter launch)
    const float c = pr_t ? 1.0f : (float)(1.4426950408889634074 / (double)temperature);
    if (!(c > 0.0f) || !isfinite(c)) return SPECDEC_EINVAL;
    if (team < 0 || team > kTreeMaxTeam) return SPECDEC_EINVAL;
    TreeWs w;
    if (!tree_ws(B, N, V, dtype, top_k, top_p, per_request, &w)) return SPECDEC_EINVAL;
    const size_t rows = 2 * ((size_t)N + B);
    if (w.sel.filter && rows * w.sel.nchunks > 0x7fffffffu) return SPECDEC_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 15) != 0 || workspace_bytes < w.total)
        return SPECDEC_EWORKSPACE;
    int G = team;
    if (G == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return SPECDEC_EHIP;
        G = cus / B;
        G = G < 1 ? 1 : (G > kTreeMaxTeam ? kTreeMaxTeam : G);
        if (G > w.nchunk) G = w.nchunk;
    }
    const int es = dtype == SPECDEC_BF16 ? 2 : 4;
    const bool vec = ((size_t)V * es) % 16 == 0 && ((uintptr_t)target_logits & 15) == 0 &&
                     ((uintptr_t)draft_logits & 15) == 0;
    TreeArgs a;
    a.tgt = reinterpret_cast<const uint8_t*>(target_logits);
    a.dft = reinterpret_cast<const uint8_t*>(draft_logits);
    a.tokens = tree_tokens;
    a.parent = tree_parent;
    a.cu = cu_nodes;
    a.u_acc = u_accept;
    a.u_smp = u_sample;
    a.B = B;
    a.N = N;
    a.max_nodes = max_nodes;
    a.V = V;
    a.c = c;
    a.out_tokens = out_tokens;
    a.nodes_out = accepted_nodes;
    a.num_acc = num_accepted;
    a.num_emit = num_emitted;
    a.err_word = err_word;
    a.req_flags = req_flags;
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    a.ctr = reinterpret_cast<int*>(ws);
    a.ring = reinterpret_cast<double*>(ws + w.ctr_bytes);
    a.nchunk = w.nchunk;
    a.nsub = w.nsub;
    a.slot = w.slot;
    a.team = G;
    // testing only: a smaller bound on the team's wait forces SPECDEC_ERR_TEAM from the host
    a.spin_limit = kTreeSpinLimit;
    a.thr = w.sel.filter ? reinterpret_cast<const float*>(ws + w.sel.thr) : nullptr;
    a.part = w.sel.filter ? reinterpret_cast<const RowPartial*>(ws + w.sel.part) : nullptr;
    a.rows = N + B;
    const bool listed = w.sel.filter && w.sel.tk_listed;
    a.kn = listed ? reinterpret_cast<const int*>(ws + w.sel.tk_kn) : nullptr;
    a.ktok = listed ? reinterpret_cast<const uint32_t*>(ws + w.sel.tk_ktok) : nullptr;
    a.kkey = listed ? reinterpret_cast<const uint16_t*>(ws + w.sel.tk_kkey) : nullptr;
    a.rpar = w.sel.pr ? reinterpret_cast<const RowParams*>(ws + w.sel.rpar) : nullptr;
    if (const char* lim = getenv("SPECDEC_TREE_SPIN_LIMIT")) {
        char* end = nullptr;
        const long v = strtol(lim, &end, 10);
        if (end != lim && *end == '\0' && v >= 0 && v <= kTreeSpinLimit) a.spin_limit = (int)v;
    }
    const int nctr = B * kTreeCtrStride;
    const int grid = (B + 7) / 8 * 8 * G;
    (void)hipGetLastError();
    int* need = reinterpret_cast<int*>(ws + w.need);
    const int nneed = w.sel.filter ? N + B : 0;
    const int nreset = nctr > nneed ? nctr : nneed;
    hipLaunchKernelGGL(k_tree_reset, dim3((nreset + 255) / 256), dim3(256), 0, stream, a.ctr, nctr,
                       need, nneed);
    if (w.sel.filter && N > 0)
        hipLaunchKernelGGL(k_tree_mark, dim3((N + 255) / 256), dim3(256), 0, stream, cu_nodes,
                           tree_parent, B, N, need);
    if (w.sel.pr) {
        ParamArgs pa{};
        pa.cu = cu_nodes;
        pa.B = B;
        pa.K = N;
        pa.V = V;
        pa.temp = per_request->temperature;
        pa.topk = per_request->top_k;
        pa.topp = per_request->top_p;
        pa.T = temperature;
        pa.top_k = top_k;
        pa.top_p = top_p;
        pa.top_k_max = per_request->top_k ? per_request->top_k_max : top_k;
        pa.kc = w.sel.kc;
        pa.tree = 1;
        pa.out = reinterpret_cast<RowParams*>(ws + w.sel.rpar);
        hipLaunchKernelGGL(k_tree_params, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                           pa, (int)rows);
    }
    if (w.sel.filter && w.sel.pr) {
        const TopkArgs ta = topk_args(a.tgt, a.dft, N + B, V, top_p, c, w.sel, ws);
        const dim3 g((unsigned)(rows * w.sel.nchunks));
        if (dtype == SPECDEC_BF16) {
            if (vec) hipLaunchKernelGGL((k_tree_select_pr<true, true>), g, dim3(kTkNT), 0, stream, ta, need);
            else hipLaunchKernelGGL((k_tree_select_pr<true, false>), g, dim3(kTkNT), 0, stream, ta, need);
            hipLaunchKernelGGL((k_tree_merge_pr<true, kMergeNT>), dim3((unsigned)rows), dim3(kMergeNT), 0, stream, ta, need);
        } else {
            if (vec) hipLaunchKernelGGL((k_tree_select_pr<false, true>), g, dim3(kTkNT), 0, stream, ta, need);
            else hipLaunchKernelGGL((k_tree_select_pr<false, false>), g, dim3(kTkNT), 0, stream, ta, need);
            hipLaunchKernelGGL((k_tree_merge_pr<false, kMergeNT>), dim3((unsigned)rows), dim3(kMergeNT), 0, stream, ta, need);
        }
    } else if (w.sel.filter) {
        const TopkArgs ta = topk_args(a.tgt, a.dft, N + B, V, top_p, c, w.sel, ws);
        const dim3 g((unsigned)(rows * w.sel.nchunks));
        if (!ta.generic) {
            const bool p2 = w.sel.topp_mode == 2;
            if (dtype == SPECDEC_BF16) {
                if (vec) {
                    if (p2) hipLaunchKernelGGL((k_tree_topp<true>), g, dim3(kTkNT), 0, stream, ta, need);
                    else hipLaunchKernelGGL((k_tree_select<true, true, false>), g, dim3(kTkNT), 0, stream, ta, need);
                } else {
                    if (p2) hipLaunchKernelGGL((k_tree_select<true, false, true>), g, dim3(kTkNT), 0, stream, ta, need);
                    else hipLaunchKernelGGL((k_tree_select<true, false, false>), g, dim3(kTkNT), 0, stream, ta, need);
                }
            } else {
                if (vec) {
                    if (p2) hipLaunchKernelGGL((k_tree_topp<false>), g, dim3(kTkNT), 0, stream, ta, need);
                    else hipLaunchKernelGGL((k_tree_select<false, true, false>), g, dim3(kTkNT), 0, stream, ta, need);
                } else {
                    if (p2) hipLaunchKernelGGL((k_tree_select<false, false, true>), g, dim3(kTkNT), 0, stream, ta, need);
                    else hipLaunchKernelGGL((k_tree_select<false, false, false>), g, dim3(kTkNT), 0, stream, ta, need);
                }
            }
        }
        if (dtype == SPECDEC_BF16)
            hipLaunchKernelGGL((k_tree_merge<true, kMergeNT>), dim3((unsigned)rows), dim3(kMergeNT), 0, stream, ta, need);
        else
            hipLaunchKernelGGL((k_tree_merge<false, kMergeNT>), dim3((unsigned)rows), dim3(kMergeNT), 0, stream, ta, need);
    }
    if (dtype == SPECDEC_BF16) {
        if (vec) hipLaunchKernelGGL((k_tree_verify<true, true>), dim3(grid), dim3(kTreeNT), 0, stream, a);
        else hipLaunchKernelGGL((k_tree_verify<true, false>), dim3(grid), dim3(kTreeNT), 0, stream, a);
    } else {
        if (vec) hipLaunchKernelGGL((k_tree_verify<false, true>), dim3(grid), dim3(kTreeNT), 0, stream, a);
        else hipLaunchKernelGGL((k_tree_verify<false, false>), dim3(grid), dim3(kTreeNT), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}
