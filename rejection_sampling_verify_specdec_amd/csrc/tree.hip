// Verification of draft trees for gfx950: one 1024-thread workgroup per request walks its
// tree (tree_dev.h). The cache step that keeps the accepted path is kv_tree_commit
// (kv.hip).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "tree_dev.h"

namespace sd {

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kTreeNT) void k_tree_verify(TreeArgs a) {
    tree_walk_body<BF16, VEC>(a, blockIdx.x);
}

}  // namespace sd

extern "C" int specdec_tree_verify(const void* target_logits, const void* draft_logits,
                                   int32_t dtype, const int32_t* tree_tokens,
                                   const int32_t* tree_parent, const int32_t* cu_nodes,
                                   const float* u_accept, const float* u_sample, int32_t B,
                                   int32_t N, int32_t max_nodes, int32_t V, float temperature,
                                   int32_t* out_tokens, int32_t* accepted_nodes,
                                   int32_t* num_accepted, int32_t* num_emitted,
                                   int32_t* err_word, int32_t* req_flags, hipStream_t stream) {
    using namespace sd;
    if (B < 1 || N < 0 || V < 1 || V > SPECDEC_MAX_V || max_nodes < 0 ||
        max_nodes > SPECDEC_MAX_TREE)
        return SPECDEC_EINVAL;
    if ((long long)N > (long long)B * max_nodes) return SPECDEC_EINVAL;
    if (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) return SPECDEC_EINVAL;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return SPECDEC_EINVAL;
    if (!target_logits || !draft_logits || !cu_nodes || !u_sample || !out_tokens ||
        !num_accepted || !num_emitted || !err_word)
        return SPECDEC_EINVAL;
    if (N > 0 && (!tree_tokens || !tree_parent || !u_accept || !accepted_nodes))
        return SPECDEC_EINVAL;
    const float c = (float)(1.4426950408889634074 / (double)temperature);   // log2(e) / T
    if (!(c > 0.0f) || !isfinite(c)) return SPECDEC_EINVAL;
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
    (void)hipGetLastError();
    if (dtype == SPECDEC_BF16) {
        if (vec) hipLaunchKernelGGL((k_tree_verify<true, true>), dim3(B), dim3(kTreeNT), 0, stream, a);
        else hipLaunchKernelGGL((k_tree_verify<true, false>), dim3(B), dim3(kTreeNT), 0, stream, a);
    } else {
        if (vec) hipLaunchKernelGGL((k_tree_verify<false, true>), dim3(B), dim3(kTreeNT), 0, stream, a);
        else hipLaunchKernelGGL((k_tree_verify<false, false>), dim3(B), dim3(kTreeNT), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}
