// Batched speculative-decoding verification for gfx950 (MI355X).
//
// What is computed follows "Speculative decoding: accelerate LLM generation without
// changing its answers", section 2 "Draft, verify, correct" (accept y_i with probability
// min(1, p_i(y_i)/q_i(y_i)) left to right, replacement from normalize(max(0, p_j - q_j))
// at the first rejection j, bonus token from p_{k+1} when all are accepted), with the
// decoding transform (temperature, top-k, top-p) applied identically to target and draft
// rows (sections 3 and 4) and a max-subtracted (stable) softmax (same page, section 6).
//
// Pipeline on one stream, per call (four kernels, five with top-k or top-p):
//   k_row_stats   every target and draft row is streamed once in 16K-element chunks with
//                 128-bit loads; each workgroup writes the chunk max m_c and
//                 S_c = sum exp2((z - m_c) * c), c = log2(e) / T, as an fp32/fp64 pair.
//   k_topk_chunks (top-k or top-p, replaces k_row_stats) the same chunks, held in
//                 registers as order-preserving keys: each workgroup writes the few tokens
//                 that can be in the row's top-k set (a bound from its per-thread maxima);
//                 for top-p alone, the chunk's top k_c tokens plus its max and exp-sum
//                 (k_topp_chunks, the same body at eight waves per SIMD).
//   k_topk_merge  one workgroup per row: exact top-k threshold over the chunks'
//                 candidates, then the nucleus boundary (top-p) in fixed-point mass, both
//                 from the token count on each key when the candidates' keys span fewer
//                 than 1024 values (bf16 rows), else from digit histograms; max, kept
//                 count and kept-set sum; rows the candidates do not cover take full passes
//                 over the row.
//   k_decide      one workgroup per request: combines the row partials in fp64, evaluates
//                 p_i(y_i), q_i(y_i) in fp64 and the accept test u * q < p left to right,
//                 finds the first rejection, publishes the accepted tokens and stores the
//                 parameters of the one row pair (or bonus row) still to be sampled.
//   k_part        one workgroup per (request, 8192-token chunk): sums of the sampling
//                 weights over the four 2048-token sub-chunks of that row (pair). Rows
//                 after the first rejection are never read again (ragged early exit).
//                 A bf16 top-k request draws here, from its row's kept-token list.
//   k_pick        one workgroup per request: W from the sub-chunk sums, t = u * W, the
//                 sub-chunk holding t scanned in ascending token order (LDS prefix scan)
//                 for the smallest x with C(x) > t.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

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

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_row_stats(const uint8_t* __restrict__ tgt,
                                                   const uint8_t* __restrict__ dft,
                                                   int rows_t, int V, int nchunks, float c,
                                                   RowPartial* __restrict__ part,
                                                   const RowParams* __restrict__ rpar) {
    row_stats_body<BF16, VEC>(tgt, dft, rows_t, V, nchunks, c, part, blockIdx.x, rpar);
}

template <bool BF16, bool VEC, bool P2>
__global__ __launch_bounds__(kTkNT) void k_topk_chunks(TopkArgs a) {
    topk_chunk_body<BF16, VEC, P2 ? 1 : 0>(a, blockIdx.x / a.nchunks, blockIdx.x % a.nchunks,
                                          ChunkSel{a.top_k, a.c, P2});
}

// top-p alone over 16-byte loads, held to 64 VGPRs: eight waves per SIMD hide its loads
// better than the fewer instructions of a larger register budget would pay
template <bool BF16>
__global__ __launch_bounds__(kTkNT) __attribute__((amdgpu_waves_per_eu(8))) void
k_topp_chunks(TopkArgs a) {
    topk_chunk_body<BF16, true, 1>(a, blockIdx.x / a.nchunks, blockIdx.x % a.nchunks,
                                   ChunkSel{a.top_k, a.c, true});
}

template <bool BF16, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(5))) void k_topk_merge(TopkArgs a) {
    topk_merge_body<BF16, NT>(a, blockIdx.x, RowSel{a.top_k, a.topp_mode, a.top_p, a.c});
}

// per-request parameters: each row's transform, then the chunks and merges that read it
__global__ __launch_bounds__(256) void k_row_params(ParamArgs a, int rows) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r < rows) row_params_one(a, r);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kTkNT) void k_chunks_pr(TopkArgs a) {
    chunk_pr_body<BF16, VEC>(a, blockIdx.x / a.nchunks, blockIdx.x % a.nchunks);
}

template <bool BF16, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(5))) void k_merge_pr(TopkArgs a) {
    merge_pr_body<BF16, NT>(a, blockIdx.x);
}

template <bool BF16>
__global__ __launch_bounds__(kDecideNT) void k_decide(SampleArgs a) {
    decide_kernel_body<BF16, kDecideNT>(a, blockIdx.x);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kPartNT) void k_part(SampleArgs a) {
    part_body<BF16, VEC, kPartNT>(a, blockIdx.x / a.nch, blockIdx.x % a.nch);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kPickNT) void k_pick(SampleArgs a) {
    pick_body<BF16, VEC, kPickNT>(a, blockIdx.x);
}

// Early exit: the statistics of position p's rows of the requests still live at p
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_pass(SampleArgs a, RowPartial* __restrict__ part, int p) {
    pass_body<BF16, VEC>(a, part, p, blockIdx.x);
}

// Early exit, the last statistics launch: every row from position p on of the requests
// still live at p
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_tail(SampleArgs a, RowPartial* __restrict__ part, int p) {
    tail_body<BF16, VEC>(a, part, p, blockIdx.x);
}

// Early exit with a top-k / top-p transform: the chunk select of position p's rows (of every
// later row for the tail launch) of the live requests, then their merge
template <bool BF16, bool VEC, int P2>
__global__ __launch_bounds__(kTkNT) void k_fpass(SampleArgs a, TopkArgs ta, int p) {
    fpass_body<BF16, VEC, P2>(a, ta, p, blockIdx.x);
}

template <bool BF16, bool VEC, int P2>
__global__ __launch_bounds__(kTkNT) void k_ftail(SampleArgs a, TopkArgs ta, int p) {
    ftail_body<BF16, VEC, P2>(a, ta, p, blockIdx.x);
}

template <bool BF16, bool PR>
__global__ __launch_bounds__(kMergeNT) __attribute__((amdgpu_waves_per_eu(5))) void k_fmerge(
    SampleArgs a, TopkArgs ta, int p, int tail) {
    fmerge_body<BF16, kMergeNT, PR>(a, ta, p, blockIdx.x, tail != 0);
}

template <bool BF16, bool VEC, int P2>
static void launch_early_filtered(int B, int K, int max_k, const TopkArgs& ta,
                                  const SampleArgs& sa, const ParamArgs& pa, hipStream_t st) {
    constexpr bool PR = P2 == 2;
    if (PR) {
        const int rows = 2 * K + B;
        hipLaunchKernelGGL(k_row_params, dim3((unsigned)(rows + 255) / 256), dim3(256), 0, st, pa,
                           rows);
    }
    for (int q = 0; q <= max_k && q < kEarlyCut; ++q) {
        hipLaunchKernelGGL((k_fpass<BF16, VEC, P2>), dim3((unsigned)B * 2u * (unsigned)ta.nchunks),
                           dim3(kTkNT), 0, st, sa, ta, q);
        hipLaunchKernelGGL((k_fmerge<BF16, PR>), dim3((unsigned)B * 2u), dim3(kMergeNT), 0, st,
                           sa, ta, q, 0);
    }
    if (max_k >= kEarlyCut) {
        const unsigned per = (unsigned)early_tail_slots(max_k, kEarlyCut);
        hipLaunchKernelGGL((k_ftail<BF16, VEC, P2>), dim3((unsigned)B * per * (unsigned)ta.nchunks),
                           dim3(kTkNT), 0, st, sa, ta, kEarlyCut);
        hipLaunchKernelGGL((k_fmerge<BF16, PR>), dim3((unsigned)B * per), dim3(kMergeNT), 0, st,
                           sa, ta, kEarlyCut, 1);
    }
}

template <bool BF16, bool VEC>
static void launch_all(const uint8_t* tgt, const uint8_t* dft, int B, int K, int V,
                       float top_p, float c, const WsPlan& p, uint8_t* ws, SampleArgs sa,
                       const ParamArgs& pa, const specdec_debug* dbg, hipStream_t st,
                       bool early, int max_k) {
    const int rows = 2 * K + B;
    RowPartial* part = reinterpret_cast<RowPartial*>(ws + p.part);
    // optional timing events are attached to the statistics launch itself
    hipEvent_t e0 = dbg ? dbg->ev_stats_begin : nullptr;
    hipEvent_t e1 = dbg ? dbg->ev_stats_end : nullptr;
    if (early && p.filter) {
        // the same positions, each a chunk-select and a merge launch
        const TopkArgs ta = topk_args(tgt, dft, K + B, V, top_p, c, p, ws);
        if (e0) (void)hipEventRecord(e0, st);
        if (p.pr) launch_early_filtered<BF16, VEC, 2>(B, K, max_k, ta, sa, pa, st);
        else if (p.topp_mode == 2) launch_early_filtered<BF16, VEC, 1>(B, K, max_k, ta, sa, pa, st);
        else launch_early_filtered<BF16, VEC, 0>(B, K, max_k, ta, sa, pa, st);
        if (e1) (void)hipEventRecord(e1, st);
    } else if (early) {
        // one launch per position up to kEarlyCut, then one for the rest; the events
        // bracket them all
        if (p.pr_plain)
            hipLaunchKernelGGL(k_row_params, dim3((unsigned)(rows + 255) / 256), dim3(256), 0, st,
                               pa, rows);
        if (e0) (void)hipEventRecord(e0, st);
        for (int q = 0; q <= max_k && q < kEarlyCut; ++q)
            hipLaunchKernelGGL((k_pass<BF16, VEC>), dim3((unsigned)B * 2u * (unsigned)p.nchunks),
                               dim3(kNT), 0, st, sa, part, q);
        if (max_k >= kEarlyCut)
            hipLaunchKernelGGL((k_tail<BF16, VEC>), dim3((unsigned)B * (unsigned)p.nchunks),
                               dim3(kNT), 0, st, sa, part, kEarlyCut);
        if (e1) (void)hipEventRecord(e1, st);
    } else if (p.pr_plain) {
        hipLaunchKernelGGL(k_row_params, dim3((unsigned)(rows + 255) / 256), dim3(256), 0, st, pa,
                           rows);
        hipExtLaunchKernelGGL((k_row_stats<BF16, VEC>), dim3((unsigned)rows * p.nchunks), dim3(kNT),
                              0, st, e0, e1, 0, tgt, dft, K + B, V, p.nchunks, c, part,
                              reinterpret_cast<const RowParams*>(ws + p.rpar));
    } else if (p.pr) {
        const TopkArgs ta = topk_args(tgt, dft, K + B, V, top_p, c, p, ws);
        hipLaunchKernelGGL(k_row_params, dim3((unsigned)(rows + 255) / 256), dim3(256), 0, st, pa,
                           rows);
        hipExtLaunchKernelGGL((k_chunks_pr<BF16, VEC>), dim3((unsigned)rows * p.nchunks),
                              dim3(kTkNT), 0, st, e0, e1, 0, ta);
        hipLaunchKernelGGL((k_merge_pr<BF16, kMergeNT>), dim3(rows), dim3(kMergeNT), 0, st, ta);
    } else if (p.filter) {
        const TopkArgs ta = topk_args(tgt, dft, K + B, V, top_p, c, p, ws);
        if (!ta.generic) {
            if (p.topp_mode == 2 && VEC)
                hipExtLaunchKernelGGL((k_topp_chunks<BF16>), dim3((unsigned)rows * p.nchunks),
                                      dim3(kTkNT), 0, st, e0, e1, 0, ta);
            else if (p.topp_mode == 2)
                hipExtLaunchKernelGGL((k_topk_chunks<BF16, VEC, true>),
                                      dim3((unsigned)rows * p.nchunks), dim3(kTkNT), 0, st, e0, e1,
                                      0, ta);
            else
                hipExtLaunchKernelGGL((k_topk_chunks<BF16, VEC, false>),
                                      dim3((unsigned)rows * p.nchunks), dim3(kTkNT), 0, st, e0, e1,
                                      0, ta);
            e0 = e1 = nullptr;
        }
        hipExtLaunchKernelGGL((k_topk_merge<BF16, kMergeNT>), dim3(rows), dim3(kMergeNT), 0, st,
                              e0, e1, 0, ta);
    } else {
        hipExtLaunchKernelGGL((k_row_stats<BF16, VEC>), dim3((unsigned)rows * p.nchunks), dim3(kNT),
                              0, st, e0, e1, 0, tgt, dft, K + B, V, p.nchunks, c, part,
                              (const RowParams*)nullptr);
    }
    if (dbg && dbg->ev_stats_done) (void)hipEventRecord(dbg->ev_stats_done, st);
    hipLaunchKernelGGL((k_decide<BF16>), dim3(B), dim3(kDecideNT), 0, st, sa);
    hipLaunchKernelGGL((k_part<BF16, VEC>), dim3((unsigned)B * p.nch), dim3(kPartNT), 0, st, sa);
    hipLaunchKernelGGL((k_pick<BF16, VEC>), dim3(B), dim3(kPickNT), 0, st, sa);
    if (sa.prec && K > 0) {
        // acceptance analytics: residual mass of every proposal position, then beta and E[A]
        hipLaunchKernelGGL((k_accept_part<BF16, VEC>), dim3((unsigned)K * p.nch), dim3(kPartNT), 0,
                           st, sa);
        hipLaunchKernelGGL((k_accept_final<BF16>), dim3(B), dim3(kWave), 0, st, sa);
    } else if (sa.prec) {
        hipLaunchKernelGGL((k_accept_final<BF16>), dim3(B), dim3(kWave), 0, st, sa);
    }
}

}  // namespace sd

extern "C" size_t specdec_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype,
                                                int32_t top_k, float top_p,
                                                const specdec_params* per_request) {
    if (B < 1 || K < 0 || V < 1 || V > SPECDEC_MAX_V || (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) ||
        (top_p != top_p && !(per_request && per_request->top_p)) ||
        (per_request && per_request->top_k && per_request->top_k_max < 0))
        return 0;
    return sd::plan_ws(B, K, V, dtype, top_k, top_p, per_request).total;
}

static int verify_entry(bool early, const void* target_logits, const void* draft_logits,
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
    const WsPlan p = plan_ws(B, K, V, dtype, top_k, top_p, per_request);
    if ((size_t)(2 * (size_t)K + B) * p.nchunks > 0x7fffffffu ||
        (size_t)K * p.nch > 0x7fffffffu || V > SPECDEC_MAX_V ||
        (early && (size_t)2 * B * p.nchunks > 0x7fffffffu) ||
        (early && max_k >= kEarlyCut &&
         (size_t)B * early_tail_slots(max_k, kEarlyCut) * p.nchunks > 0x7fffffffu))
        return SPECDEC_EINVAL;
    if (!workspace || workspace_bytes < p.total || ((uintptr_t)workspace & 15))
        return SPECDEC_EWORKSPACE;

    const double c64 = 1.4426950408889634074 / (double)temperature;   // log2(e) / T
    const float c = pr_t ? 1.0f : (float)c64;
    if (!(c > 0.0f) || !isfinite(c)) return SPECDEC_EINVAL;
    const int es = dtype == SPECDEC_BF16 ? 2 : 4;
    const bool vec = ((size_t)V * es) % 16 == 0 && ((uintptr_t)target_logits & 15) == 0 &&
                     (K == 0 || ((uintptr_t)draft_logits & 15) == 0);
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    const uint8_t* tgt = reinterpret_cast<const uint8_t*>(target_logits);
    const uint8_t* dft = reinterpret_cast<const uint8_t*>(K > 0 ? draft_logits : target_logits);

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
    sa.live = reinterpret_cast<int*>(ws + p.live);
    sa.rpar = p.pr ? reinterpret_cast<const RowParams*>(ws + p.rpar) : nullptr;
    sa.part = reinterpret_cast<const RowPartial*>(ws + p.part);
    sa.row_thr = reinterpret_cast<const float*>(ws + p.thr);
    sa.rec = reinterpret_cast<Decision*>(ws + p.rec);
    sa.wsum = reinterpret_cast<double*>(ws + p.wsum);
    sa.kn = p.tk_listed ? reinterpret_cast<const int*>(ws + p.tk_kn) : nullptr;
    sa.ktok = p.tk_listed ? reinterpret_cast<const uint32_t*>(ws + p.tk_ktok) : nullptr;
    sa.kkey = p.tk_listed ? reinterpret_cast<const uint16_t*>(ws + p.tk_kkey) : nullptr;
    sa.out_tokens = out_tokens;
    sa.num_acc = num_accepted;
    sa.num_emit = num_emitted;
    sa.err_word = err_word;
    if (dbg) {
        sa.dbg = *dbg;
    } else {
        sa.dbg = specdec_debug{};
    }
    const bool analytics = dbg && (dbg->accept_prob || dbg->expected_emitted);
    sa.prec = analytics ? reinterpret_cast<Decision*>(ws + p.prec) : nullptr;
    sa.wacc = analytics ? reinterpret_cast<double*>(ws + p.wacc) : nullptr;

    ParamArgs pa{};
    if (p.pr) pa = param_args(cu_draft, B, K, V, temperature, top_k, top_p, per_request, p, ws);

    (void)hipGetLastError();
    if (dtype == SPECDEC_BF16) {
        if (vec) launch_all<true, true>(tgt, dft, B, K, V, top_p, c, p, ws, sa, pa, dbg, stream, early, max_k);
        else launch_all<true, false>(tgt, dft, B, K, V, top_p, c, p, ws, sa, pa, dbg, stream, early, max_k);
    } else {
        if (vec) launch_all<false, true>(tgt, dft, B, K, V, top_p, c, p, ws, sa, pa, dbg, stream, early, max_k);
        else launch_all<false, false>(tgt, dft, B, K, V, top_p, c, p, ws, sa, pa, dbg, stream, early, max_k);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

extern "C" int specdec_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                              const int32_t* draft_tokens, const int32_t* cu_draft,
                              const float* u_accept, const float* u_sample, int32_t B, int32_t K,
                              int32_t max_k, int32_t V, float temperature, int32_t top_k,
                              float top_p, const specdec_params* per_request,
                              int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                              int32_t* err_word, const specdec_debug* dbg, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    return verify_entry(false, target_logits, draft_logits, dtype, draft_tokens, cu_draft,
                        u_accept, u_sample, B, K, max_k, V, temperature, top_k, top_p,
                        per_request, out_tokens, num_accepted, num_emitted, err_word, dbg,
                        workspace, workspace_bytes, stream);
}

extern "C" int specdec_verify_early_exit(const void* target_logits, const void* draft_logits,
                                         int32_t dtype, const int32_t* draft_tokens,
                                         const int32_t* cu_draft, const float* u_accept,
                                         const float* u_sample, int32_t B, int32_t K,
                                         int32_t max_k, int32_t V, float temperature,
                                         int32_t top_k, float top_p,
                                         const specdec_params* per_request, int32_t* out_tokens,
                                         int32_t* num_accepted, int32_t* num_emitted,
                                         int32_t* err_word, const specdec_debug* dbg,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
    return verify_entry(true, target_logits, draft_logits, dtype, draft_tokens, cu_draft,
                        u_accept, u_sample, B, K, max_k, V, temperature, top_k, top_p,
                        per_request, out_tokens, num_accepted, num_emitted, err_word, dbg,
                        workspace, workspace_bytes, stream);
}

extern "C" const char* specdec_status_string(int status) {
    switch (status) {
        case SPECDEC_OK: return "ok";
        case SPECDEC_EINVAL: return "invalid argument";
        case SPECDEC_EHIP: return "HIP runtime error";
        case SPECDEC_EWORKSPACE: return "workspace missing, misaligned or too small";
        case SPECDEC_ESCRATCH:
            return "the call needs more scratch than the static array holds; use the entry "
                   "point that takes a workspace";
        default: return "unknown status";
    }
}
