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

#include "common.h"
#include "specdec.h"

namespace sd {

constexpr int kKvNT = 1024;      // single-workgroup bookkeeping kernels
constexpr int kKvRPT = SPECDEC_MAX_KV_BATCH / kKvNT;   // requests per thread
constexpr int kScNT = 256;       // scatter workgroup
constexpr int kScMaxTok = 16;    // tokens per scatter workgroup (for small rows)
constexpr int kEvCap = 2048;     // rollback events per window
constexpr int kEvPT = kEvCap / kKvNT;

struct KvArgs {
    uint8_t* pool;
    int L, H, D, bs, NB, MBR;
    int* tables;
    int* seq_lens;
    int* refcount;
    int* free_list;
    int* free_count;
    int* state;
};

// append workspace: [0] status (0 applied, 1 rejected), [1] copy-on-write entries left
// for the scatter (stored from the front of the entry array), [2] entries whose source
// block another request writes in place in the same batch (stored from the back; copied
// by k_kv_alloc itself so the copy reads before the scatter writes), [3] unused, then
// B entries (src block, dst block, slots, b), then N int64 destination rows (physical
// block * block_size + slot) of the new entries, -1 where the block id is corrupt.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct CowEntry {
    int src, dst, nslots, b;
};

SD_DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }

SD_DEV void copy_slots(const KvArgs& a, int src, int dst, int nslots, int tid, int nt) {
    // all layers, K and V: slots [0, nslots) of block src -> block dst
    const size_t ub = (size_t)a.H * a.D * 2;
    const size_t per_blk = (size_t)a.bs * ub;
    const size_t vec_per = (size_t)nslots * ub / 16;
    for (int lk = 0; lk < a.L * 2; ++lk) {
        const uint4* s = reinterpret_cast<const uint4*>(a.pool + ((size_t)lk * a.NB + src) * per_blk);
        uint4* d = reinterpret_cast<uint4*>(a.pool + ((size_t)lk * a.NB + dst) * per_blk);
        for (size_t i = tid; i < vec_per; i += nt) d[i] = s[i];
    }
}

// Requests are spread over the workgroup with stride kKvNT (request b = round * kKvNT +
// thread), so a batch of up to kKvNT requests costs one pass of dependent loads; ordered
// quantities (pop positions) come from per-round exclusive scans with a running carry.
__global__ __launch_bounds__(kKvNT) void k_kv_alloc(KvArgs a, const int* __restrict__ cu_new,
                                                    int B, int N, int* __restrict__ ws) {
    __shared__ int redi[kKvNT / kWave];
    __shared__ int s_pot_b[SPECDEC_MAX_KV_BATCH];
    __shared__ int s_pot_X[SPECDEC_MAX_KV_BATCH];
    const int tid = threadIdx.x;
    const int rounds = (B + kKvNT - 1) / kKvNT;
    const int fc = *a.free_count;
    int s[kKvRPT], n[kKvRPT], X[kKvRPT], r0[kKvRPT];
    int bad = 0;
    if (tid == 0 && (cu_new[0] != 0 || cu_new[B] != N)) bad = 1;
#pragma unroll
    for (int i = 0; i < kKvRPT; ++i) {
        const int b = i * kKvNT + tid;
        s[i] = n[i] = 0;
        X[i] = -1;
        r0[i] = 0;
        if (b >= B) continue;
        s[i] = a.seq_lens[b];
        n[i] = cu_new[b + 1] - cu_new[b];
        if (n[i] < 0 || s[i] < 0 || (long long)s[i] + n[i] > (long long)a.MBR * a.bs) {
            bad = 1;
            continue;
        }
        if (n[i] > 0 && s[i] % a.bs != 0) {
            X[i] = a.tables[(size_t)b * a.MBR + s[i] / a.bs];
            if (X[i] < 0 || X[i] >= a.NB) {
                bad = 1;
                continue;
            }
            r0[i] = a.refcount[X[i]];
        }
    }
    bad = block_max_i<kKvNT>(bad, redi);
    if (bad) {
        if (tid == 0) {
            ws[0] = 1;
            ws[1] = 0;
            atomicOr(a.state, KV_ERR_APPEND | KV_APPEND_REJECTED);
        }
        return;
    }
    // shared partial blocks receiving entries, listed in request order
    int P = 0;
    for (int i = 0; i < rounds; ++i) {
        const int pot = (X[i] >= 0 && r0[i] > 1) ? 1 : 0;
        int tot;
        const int pos = P + block_excl_scan_i<kKvNT>(pot, redi, &tot);
        if (pot) {
            s_pot_b[pos] = i * kKvNT + tid;
            s_pot_X[pos] = X[i];
        }
        P += tot;
    }
    if (tid == 0) {
        ws[1] = 0;
        ws[2] = 0;
    }
    __syncthreads();
    // copy-on-write: the i-th sharer (in request order) of block X copies iff i < r0 - 1,
    // which is what processing the batch in order with live refcounts gives
    int cow[kKvRPT], conflict[kKvRPT], need[kKvRPT];
#pragma unroll
    for (int i = 0; i < kKvRPT; ++i) {
        const int b = i * kKvNT + tid;
        cow[i] = conflict[i] = need[i] = 0;
        if (b >= B) continue;
        if (X[i] >= 0 && r0[i] > 1) {
            int rank = 0, cnt = 0;
            for (int j = 0; j < P; ++j) {
                if (s_pot_X[j] == X[i]) {
                    ++cnt;
                    if (s_pot_b[j] < b) ++rank;
                }
            }
            cow[i] = rank < r0[i] - 1;
            // another sharer writes X in place in this batch: copy before the scatter
            conflict[i] = cow[i] && cnt > r0[i] - 1;
        }
        if (n[i] > 0) need[i] = ceil_div(s[i] + n[i], a.bs) - ceil_div(s[i], a.bs) + cow[i];
    }
    int base[kKvRPT];
    int T = 0;
    for (int i = 0; i < rounds; ++i) {
        int tot;
        base[i] = T + block_excl_scan_i<kKvNT>(need[i], redi, &tot);
        T += tot;
    }
    if (T > fc) {
        if (tid == 0) {
            ws[0] = 1;
            atomicOr(a.state, KV_ERR_NOMEM | KV_APPEND_REJECTED);
        }
        return;
    }
    for (int i = 0; i < rounds; ++i) {
        const int b = i * kKvNT + tid;
        if (b >= B || n[i] == 0) continue;
        int p = base[i];
        int* tab = a.tables + (size_t)b * a.MBR;
        if (cow[i]) {
            const int nb = a.free_list[fc - 1 - p++];
            tab[s[i] / a.bs] = nb;
            if ((unsigned)nb < (unsigned)a.NB) {
                a.refcount[nb] = 1;
                atomicSub(&a.refcount[X[i]], 1);
                CowEntry e{X[i], nb, s[i] % a.bs, b};
                CowEntry* list = reinterpret_cast<CowEntry*>(ws + 4);
                if (conflict[i]) list[B - 1 - atomicAdd(&ws[2], 1)] = e;
                else list[atomicAdd(&ws[1], 1)] = e;
            } else {
                atomicOr(a.state, KV_ERR_APPEND);    // corrupt free list
            }
        }
        const int lb_first = ceil_div(s[i], a.bs);
        const int lb_end = ceil_div(s[i] + n[i], a.bs);
        for (int lb = lb_first; lb < lb_end; ++lb) {
            const int nb = a.free_list[fc - 1 - p++];
            tab[lb] = nb;
            if ((unsigned)nb < (unsigned)a.NB) a.refcount[nb] = 1;
            else atomicOr(a.state, KV_ERR_APPEND);  // corrupt free list
        }
        // destination rows of the request's new entries, read by the scatter
        long long* drow = reinterpret_cast<long long*>(ws + 4 + 4 * B);
        const int part_blk = (s[i] % a.bs != 0) ? tab[s[i] / a.bs] : -1;
        for (int t = 0; t < n[i]; ++t) {
            const int pos = s[i] + t;
            const int lb = pos / a.bs;
            const int blk = (lb < lb_first) ? part_blk : a.free_list[fc - 1 - (base[i] + cow[i] + (lb - lb_first))];
            drow[cu_new[b] + t] = (unsigned)blk < (unsigned)a.NB ? (long long)blk * a.bs + pos % a.bs : -1;
        }
        a.seq_lens[b] = s[i] + n[i];
    }
    __syncthreads();
    // copies whose source another request writes in place in this batch happen here,
    // before the scatter kernel starts
    const int nconf = atomicAdd(ws + 2, 0);   // atomics live in L2: read through one
    const CowEntry* list = reinterpret_cast<const CowEntry*>(ws + 4);
    for (int q = 0; q < nconf; ++q) {
        const CowEntry e = list[B - 1 - q];
        copy_slots(a, e.src, e.dst, e.nslots, tid, kKvNT);
    }
    if (tid == 0) {
        *a.free_count = fc - T;
        ws[0] = 0;
        atomicAnd(a.state, ~KV_APPEND_REJECTED);
    }
}

// tpw tokens per workgroup (tpw * lanes <= kScNT when a token row is small); each thread
// moves 16-byte pieces of token rows, reading the destination row the alloc kernel wrote.
__global__ __launch_bounds__(kScNT) void k_kv_scatter(KvArgs a, const uint8_t* __restrict__ knew,
                                                      const uint8_t* __restrict__ vnew, int B, int N,
                                                      int tpw, const int* __restrict__ ws) {
    if (ws[0] != 0) return;
    const int tid = threadIdx.x;
    const int lk = blockIdx.y;                 // layer * 2 + (0: K, 1: V)
    const int l = lk >> 1;
    const size_t ub = (size_t)a.H * a.D * 2;   // bytes of one token's row
    const int lanes = (int)(ub / 16);
    const int t0 = blockIdx.x * tpw;
    const long long* drow = reinterpret_cast<const long long*>(ws + 4 + 4 * B);
    const uint8_t* src_base = (lk & 1) ? vnew : knew;
    uint8_t* dst_base = a.pool + (size_t)lk * a.NB * a.bs * ub;
    for (int idx = tid; idx < tpw * lanes; idx += kScNT) {
        const int tok = idx / lanes, q = idx - tok * lanes;
        const int t = t0 + tok;
        if (t >= N) break;
        const long long d = drow[t];
        if (d < 0) continue;
        const u32x4* src = reinterpret_cast<const u32x4*>(src_base + ((size_t)l * N + t) * ub) + q;
        u32x4* dst = reinterpret_cast<u32x4*>(dst_base + (size_t)d * ub) + q;
        __builtin_nontemporal_store(__builtin_nontemporal_load(src), dst);
    }
    // copy-on-write copies (rare): grid-stride over (entry, layer, K/V)
    const int ncow = ws[1];
    if (ncow > 0) {
        const CowEntry* ce = reinterpret_cast<const CowEntry*>(ws + 4);
        const int nwg = gridDim.x * gridDim.y;
        const int wg = blockIdx.y * gridDim.x + blockIdx.x;
        const size_t per_blk = (size_t)a.bs * ub;
        for (int u = wg; u < ncow * a.L * 2; u += nwg) {
            const CowEntry e = ce[u / (a.L * 2)];
            const int ulk = u % (a.L * 2);
            const uint4* s = reinterpret_cast<const uint4*>(a.pool + ((size_t)ulk * a.NB + e.src) * per_blk);
            uint4* d = reinterpret_cast<uint4*>(a.pool + ((size_t)ulk * a.NB + e.dst) * per_blk);
            const size_t nv = (size_t)e.nslots * ub / 16;
            for (size_t i = tid; i < nv; i += kScNT) d[i] = s[i];
        }
    }
}

__global__ __launch_bounds__(kKvNT) void k_kv_rollback(KvArgs a, const int* __restrict__ num_acc,
                                                       const int* __restrict__ cu, int B) {
    __shared__ int redi[kKvNT / kWave];
    __shared__ int s_off[SPECDEC_MAX_KV_BATCH + 1];
    __shared__ int s_lb0[SPECDEC_MAX_KV_BATCH];
    __shared__ int s_X[kEvCap];
    __shared__ int s_b[kEvCap];
    __shared__ int s_lb[kEvCap];
    if (*a.state & KV_APPEND_REJECTED) return;
    const int tid = threadIdx.x;
    const int rounds = (B + kKvNT - 1) / kKvNT;
    int fc = *a.free_count;
    int err = 0;
    int newlen[kKvRPT], valid[kKvRPT];
    int E = 0;
#pragma unroll
    for (int i = 0; i < kKvRPT; ++i) {
        const int b = i * kKvNT + tid;
        valid[i] = 0;
        newlen[i] = 0;
        int ev = 0;
        if (b < B) {
            const int k = cu[b + 1] - cu[b], acc = num_acc[b], s = a.seq_lens[b];
            if (k < 0 || acc < 0 || acc > k || k - acc > s ||
                (long long)s > (long long)a.MBR * a.bs) {
                err = 1;
            } else {
                valid[i] = 1;
                newlen[i] = s - (k - acc);
                ev = ceil_div(s, a.bs) - ceil_div(newlen[i], a.bs);
            }
        }
        if (i < rounds) {
            int tot;
            const int off = E + block_excl_scan_i<kKvNT>(ev, redi, &tot);
            if (b < B) {
                s_off[b] = off;
                s_lb0[b] = ceil_div(newlen[i], a.bs);
            }
            E += tot;
        }
    }
    if (tid == 0) s_off[B] = E;
    __syncthreads();
    for (int w0 = 0; w0 < E; w0 += kEvCap) {
        const int nw = min(kEvCap, E - w0);
        // gather this window's events in (request, logical block) order
#pragma unroll
        for (int i = 0; i < kEvPT; ++i) {
            const int el = i * kKvNT + tid;
            if (el >= nw) continue;
            const int e = w0 + el;
            int lo = 0, hi = B;               // largest b with s_off[b] <= e
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_off[mid] <= e) lo = mid;
                else hi = mid;
            }
            const int lb = s_lb0[lo] + (e - s_off[lo]);
            s_b[el] = lo;
            s_lb[el] = lb;
            s_X[el] = a.tables[(size_t)lo * a.MBR + lb];
        }
        __syncthreads();
        int push[kEvPT], newrc[kEvPT], first[kEvPT];
#pragma unroll
        for (int i = 0; i < kEvPT; ++i) {
            const int el = i * kKvNT + tid;
            push[i] = first[i] = 0;
            newrc[i] = 0;
            if (el >= nw) continue;
            const int X = s_X[el];
            if (X < 0 || X >= a.NB) {
                err = 1;
                continue;
            }
            const int rc = a.refcount[X];
            int rank = 0, cnt = 0;
            for (int j = 0; j < nw; ++j) {
                if (s_X[j] == X) {
                    ++cnt;
                    if (j < el) ++rank;
                }
            }
            // sequentially, the events on X see rc, rc-1, ...: those that find it > 0
            // decrement, the one that reaches 0 pushes, the rest are errors
            if (rank >= rc) err = 1;
            push[i] = rc >= 1 && rank == rc - 1;
            first[i] = rank == 0;
            newrc[i] = rc - min(cnt, max(rc, 0));
        }
        // push positions follow event order (the scans also separate reads from writes)
        int pbase[kEvPT];
        int ptot = 0;
#pragma unroll
        for (int i = 0; i < kEvPT; ++i) {
            int tot;
            pbase[i] = ptot + block_excl_scan_i<kKvNT>(push[i], redi, &tot);
            ptot += tot;
        }
#pragma unroll
        for (int i = 0; i < kEvPT; ++i) {
            const int el = i * kKvNT + tid;
            if (el >= nw) continue;
            const int X = s_X[el];
            if (X >= 0 && X < a.NB) {
                if (first[i]) a.refcount[X] = newrc[i];
                if (push[i]) {
                    if (fc + pbase[i] < a.NB) a.free_list[fc + pbase[i]] = X;
                    else err = 1;                     // more frees than blocks: corrupt
                }
            }
            a.tables[(size_t)s_b[el] * a.MBR + s_lb[el]] = -1;
        }
        fc += ptot;
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kKvRPT; ++i) {
        const int b = i * kKvNT + tid;
        if (b < B && valid[i]) a.seq_lens[b] = newlen[i];
    }
    err = block_max_i<kKvNT>(err, redi);
    if (tid == 0) {
        *a.free_count = min(fc, a.NB);
        if (err) atomicOr(a.state, KV_ERR_ROLLBACK);
    }
}

static bool geometry_ok(const kv_paged_cache* c) {
    if (!c || !c->pool || !c->block_tables || !c->seq_lens || !c->refcount || !c->free_list ||
        !c->free_count || !c->state)
        return false;
    if (c->num_layers < 1 || c->num_kv_heads < 1 || c->head_dim < 1 || c->block_size < 1 ||
        c->num_blocks < 1 || c->max_blocks_per_req < 1)
        return false;
    if (((size_t)c->num_kv_heads * c->head_dim * 2) % 16 != 0) return false;
    if (((uintptr_t)c->pool & 15) != 0) return false;
    if ((long long)c->max_blocks_per_req * c->block_size > 0x7fffffffLL) return false;
    return true;
}

static KvArgs args_of(const kv_paged_cache* c) {
    KvArgs a;
    a.pool = reinterpret_cast<uint8_t*>(c->pool);
    a.L = c->num_layers;
    a.H = c->num_kv_heads;
    a.D = c->head_dim;
    a.bs = c->block_size;
    a.NB = c->num_blocks;
    a.MBR = c->max_blocks_per_req;
    a.tables = c->block_tables;
    a.seq_lens = c->seq_lens;
    a.refcount = c->refcount;
    a.free_list = c->free_list;
    a.free_count = c->free_count;
    a.state = c->state;
    return a;
}

}  // namespace sd

extern "C" size_t kv_paged_append_workspace_size(int32_t B, int32_t N) {
    if (B < 1 || N < 0) return 0;
    return 16 + (size_t)B * sizeof(sd::CowEntry) + (size_t)N * sizeof(long long);
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
    int* ws = reinterpret_cast<int*>(workspace);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_kv_alloc, dim3(1), dim3(kKvNT), 0, stream, a, cu_new, B, N, ws);
    const int lanes = (int)((size_t)a.H * a.D * 2 / 16);
    const int tpw = lanes >= kScNT ? 1 : min(kScMaxTok, kScNT / lanes);
    const unsigned tiles = (unsigned)((N + tpw - 1) / tpw);
    if (tiles > 0)
        hipLaunchKernelGGL(k_kv_scatter, dim3(tiles, (unsigned)a.L * 2), dim3(kScNT), 0, stream, a,
                           reinterpret_cast<const uint8_t*>(k_new),
                           reinterpret_cast<const uint8_t*>(v_new), B, N, tpw, ws);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

extern "C" int kv_rollback(const kv_paged_cache* cache, int32_t B, const int32_t* num_accepted,
                           const int32_t* cu_draft, hipStream_t stream) {
    using namespace sd;
    if (!geometry_ok(cache) || B < 1 || B > SPECDEC_MAX_KV_BATCH || !num_accepted || !cu_draft)
        return SPECDEC_EINVAL;
    const KvArgs a = args_of(cache);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_kv_rollback, dim3(1), dim3(kKvNT), 0, stream, a, num_accepted, cu_draft, B);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}
