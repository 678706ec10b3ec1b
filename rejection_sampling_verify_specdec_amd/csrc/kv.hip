// Paged KV cache around a speculative cycle for gfx950: provisional append and rollback.
//
// The cache contract follows "Keep cache validity aligned with the committed token
// history" (paragraphs 1-4: processed prefix plus accepted states are kept, the
// correction stays pending, block tables / ownership / reference counts decide which
// physical memory is valid, copy-on-write isolates shared prefixes) and "Walk through
// KV-cache updates when speculative decoding rejects some draft tokens" (candidate K/V are
// appended by the verifying pass; pages of rejected positions are freed afterwards).
//
// Kernels:
//   k_kv_alloc     one workgroup: validates, decides copy-on-write for shared partial
//                  blocks (rank of each sharer among the batch's sharers, so the result is
//                  the same as processing requests in order), pops blocks from the LIFO
//                  free list with an exclusive scan of per-request needs (ascending
//                  request, then logical block), all-or-nothing.
//   k_kv_scatter   moves the new entries (one H*D bf16 row per token, layer and K/V) into
//                  their slots with 128-bit loads / stores, then the copy-on-write copies.
//   k_kv_rollback  one workgroup: per request the blocks past the new length are
//                  decref'ed; for blocks referenced several times in the batch each
//                  event's rank among same-block events decides which one frees the block,
//                  and an exclusive scan of the frees gives deterministic push positions.
// No atomics decide any order: the free list and tables are a pure function of the
// inputs.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kv_dev.h"

namespace sd {

__global__ __launch_bounds__(kKvNT) void k_kv_alloc(KvArgs a, const int* __restrict__ cu_new,
                                                    int B, int N, uint8_t* __restrict__ ws) {
    alloc_body<kKvNT>(a, cu_new, 0, B, N, ws);
}

__global__ __launch_bounds__(kScNT) void k_kv_scatter(KvArgs a, const uint8_t* __restrict__ knew,
                                                      const uint8_t* __restrict__ vnew, int B,
                                                      int N, int tpw,
                                                      const uint8_t* __restrict__ ws) {
    // tile-major: consecutive workgroups take one tile across the layer / K-V planes (8%
    // faster than plane-major for the headline workload's append, measured)
    const int planes = a.L * 2;
    scatter_body<kScPPT>(a, knew, vnew, B, N, tpw, ws, blockIdx.x / planes, blockIdx.x % planes,
                         blockIdx.x, gridDim.x, kScNT);
}

__global__ __launch_bounds__(kKvNT) void k_kv_rollback(KvArgs a, const int* __restrict__ num_acc,
                                                       const int* __restrict__ cu, int B,
                                                       int draft, const int* __restrict__ tree,
                                                       int tree_n) {
    rollback_body(a, num_acc, cu, B, draft, tree, tree_n);
}

__global__ __launch_bounds__(kTreeGatherNT) void k_kv_tree_gather(KvArgs a,
                                                                  const int* __restrict__ num_acc,
                                                                  const int* __restrict__ nodes,
                                                                  const int* __restrict__ cu,
                                                                  int N) {
    tree_gather_body(a, num_acc, nodes, cu, N, blockIdx.x / (a.L * 2), blockIdx.x % (a.L * 2));
}

__global__ __launch_bounds__(kContigNT) void k_contig_check(ContigArgs a, const int* __restrict__ cu,
                                                            int B, int N) {
    contig_check_body(a, cu, B, N);
}

__global__ __launch_bounds__(256) void k_contig_copy(ContigArgs a, const uint8_t* __restrict__ knew,
                                                     const uint8_t* __restrict__ vnew,
                                                     const int* __restrict__ cu, int B, int N) {
    contig_copy_body(a, knew, vnew, cu, B, N, blockIdx.x, blockIdx.y);
}

__global__ __launch_bounds__(kContigNT) void k_contig_commit(ContigArgs a, const int* __restrict__ cu,
                                                             int B) {
    contig_commit_body(a, cu, B);
}

__global__ __launch_bounds__(kContigNT) void k_contig_rollback(ContigArgs a,
                                                               const int* __restrict__ num_acc,
                                                               const int* __restrict__ cu, int B,
                                                               int draft) {
    contig_rollback_body(a, num_acc, cu, B, draft);
}

}  // namespace sd

extern "C" int kv_contig_append(const kv_contig_cache* cache, int32_t B, const void* k_new,
                                const void* v_new, const int32_t* cu_new, int32_t N,
                                hipStream_t stream) {
    using namespace sd;
    if (!contig_ok(cache) || B < 1 || B > cache->batch || N < 0 || !cu_new) return SPECDEC_EINVAL;
    if (N > 0 && (!k_new || !v_new || ((uintptr_t)k_new & 15) || ((uintptr_t)v_new & 15)))
        return SPECDEC_EINVAL;
    if ((long long)cache->num_layers * 2 > 65535) return SPECDEC_EINVAL;
    const ContigArgs a = contig_args(cache);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_contig_check, dim3(1), dim3(kContigNT), 0, stream, a, cu_new, B, N);
    const unsigned tiles = (unsigned)((N + kContigTPW - 1) / kContigTPW);
    if (tiles > 0)
        hipLaunchKernelGGL(k_contig_copy, dim3(tiles, (unsigned)a.L * 2), dim3(256), 0, stream, a,
                           reinterpret_cast<const uint8_t*>(k_new),
                           reinterpret_cast<const uint8_t*>(v_new), cu_new, B, N);
    hipLaunchKernelGGL(k_contig_commit, dim3(1), dim3(kContigNT), 0, stream, a, cu_new, B);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

extern "C" int kv_contig_rollback(const kv_contig_cache* cache, int32_t B,
                                  const int32_t* num_accepted, const int32_t* cu_draft,
                                  int32_t draft, hipStream_t stream) {
    using namespace sd;
    if (!contig_ok(cache) || B < 1 || B > cache->batch || !num_accepted || !cu_draft ||
        (draft != 0 && draft != 1))
        return SPECDEC_EINVAL;
    const ContigArgs a = contig_args(cache);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_contig_rollback, dim3(1), dim3(kContigNT), 0, stream, a, num_accepted,
                       cu_draft, B, draft);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

extern "C" size_t kv_paged_append_workspace_size(int32_t B, int32_t N) {
    if (B < 1 || N < 0) return 0;
    return sd::append_ws_bytes(B, N);
}

extern "C" int kv_paged_append(const kv_paged_cache* cache, int32_t B, const void* k_new,
                               const void* v_new, const int32_t* cu_new, int32_t N,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    using namespace sd;
    if (!geometry_ok(cache) || B < 1 || B > SPECDEC_MAX_KV_BATCH || N < 0 || !cu_new)
        return SPECDEC_EINVAL;
    if (N > 0 && (!k_new || !v_new || ((uintptr_t)k_new & 15) || ((uintptr_t)v_new & 15)))
        return SPECDEC_EINVAL;
    if (!workspace || workspace_bytes < kv_paged_append_workspace_size(B, N) ||
        ((uintptr_t)workspace & 15))
        return SPECDEC_EWORKSPACE;
    const KvArgs a = args_of(cache);
    const int tpw = scatter_tokens_per_wg(a, kScNT, kScPPT);
    const unsigned tiles = (unsigned)((N + tpw - 1) / tpw);
    if ((size_t)tiles * a.L * 2 > 0x7fffffffu) return SPECDEC_EINVAL;
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_kv_alloc, dim3(1), dim3(kKvNT), 0, stream, a, cu_new, B, N, ws);
    if (tiles > 0)
        hipLaunchKernelGGL(k_kv_scatter, dim3(tiles * (unsigned)a.L * 2), dim3(kScNT), 0, stream, a,
                           reinterpret_cast<const uint8_t*>(k_new),
                           reinterpret_cast<const uint8_t*>(v_new), B, N, tpw, ws);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

static int rollback_call(const kv_paged_cache* cache, int32_t B, const int32_t* num_accepted,
                         const int32_t* cu_draft, hipStream_t stream, int draft) {
    using namespace sd;
    if (!geometry_ok(cache) || B < 1 || B > SPECDEC_MAX_KV_BATCH || !num_accepted || !cu_draft)
        return SPECDEC_EINVAL;
    const KvArgs a = args_of(cache);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_kv_rollback, dim3(1), dim3(kKvNT), 0, stream, a, num_accepted, cu_draft,
                       B, draft, static_cast<const int*>(nullptr), 0);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

extern "C" int kv_rollback(const kv_paged_cache* cache, int32_t B, const int32_t* num_accepted,
                           const int32_t* cu_draft, hipStream_t stream) {
    return rollback_call(cache, B, num_accepted, cu_draft, stream, 0);
}

extern "C" int kv_rollback_draft(const kv_paged_cache* cache, int32_t B,
                                 const int32_t* num_accepted, const int32_t* cu_draft,
                                 hipStream_t stream) {
    return rollback_call(cache, B, num_accepted, cu_draft, stream, 1);
}

extern "C" int kv_tree_commit(const kv_paged_cache* cache, int32_t B, const int32_t* num_accepted,
                              const int32_t* accepted_nodes, const int32_t* cu_nodes, int32_t N,
                              hipStream_t stream) {
    using namespace sd;
    if (!geometry_ok(cache) || B < 1 || B > SPECDEC_MAX_KV_BATCH || N < 0 || !num_accepted ||
        !cu_nodes || (N > 0 && !accepted_nodes))
        return SPECDEC_EINVAL;
    if ((long long)B * cache->num_layers * 2 > 0x7fffffffLL) return SPECDEC_EINVAL;
    const KvArgs a = args_of(cache);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_kv_tree_gather, dim3((unsigned)B * a.L * 2), dim3(kTreeGatherNT), 0,
                       stream, a, num_accepted, accepted_nodes, cu_nodes, N);
    hipLaunchKernelGGL(k_kv_rollback, dim3(1), dim3(kKvNT), 0, stream, a, num_accepted, cu_nodes,
                       B, 0, accepted_nodes, N);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}
