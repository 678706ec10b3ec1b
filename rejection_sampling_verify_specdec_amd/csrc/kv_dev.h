// Device-side bodies of the paged-KV kernels (gfx950), shared by the standalone
// kv_paged_append / kv_rollback launches and the fused cycle. See kv.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "specdec.h"

namespace sd {

constexpr int kKvNT = 1024;      // rollback workgroup (and the standalone allocation)
constexpr int kScNT = 256;       // standalone scatter workgroup
constexpr int kScPPT = 2;        // token rows per scatter thread in flight
constexpr int kEvCap = 2048;     // rollback events per window
constexpr int kTreeGatherNT = 128;   // tree commit gather workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

struct CowEntry {
    int src, dst, nslots, b;
};

// Append workspace layout (bytes):
//   0             int[4]: status (0 applied, 1 rejected); copy-on-write entries left for
//                 the scatter (stored from the front of the entry array); entries whose
//                 source block another request writes in place in the same batch (stored
//                 from the back, copied by the allocation itself so the copy reads before
//                 the scatter writes); unused
//   16            CowEntry[B]
//   16 + 16B      int[B] requests and int[B] blocks of the shared partial blocks receiving
//                 entries, in request order
//   16 + 24B      int4[B] per request: partial block, its refcount, copy / conflict
//                 flags, first pop index
//   16 + 40B      int64[N] destination row (block * block_size + slot) of each new entry,
//                 -1 where the block id is corrupt
static inline size_t append_ws_bytes(int B, int N) {
    return 16 + (size_t)40 * B + (size_t)8 * N;
}

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

// Allocation for an append, one workgroup of NT threads. Requests are spread with stride
// NT (request b = round * NT + thread), so a batch of up to NT requests costs one pass of
// dependent loads; ordered quantities (pop positions, the list of shared partial blocks)
// come from per-round exclusive scans with a running carry. Per-request state between
// passes lives in the workspace. cu gives the new-entry offsets, or, with derive, the
// proposal offsets from which n_b = k_b + 1 (cu_new[b] = cu[b] + b).
template <int NT>
SD_DEV void alloc_body(const KvArgs& a, const int* __restrict__ cu, int derive, int B, int N,
                       uint8_t* __restrict__ wsb) {
    __shared__ int redi[NT / kWave];
    int* ws = reinterpret_cast<int*>(wsb);
    CowEntry* list = reinterpret_cast<CowEntry*>(wsb + 16);
    int* pot_b = reinterpret_cast<int*>(wsb + 16 + (size_t)16 * B);
    int* pot_X = pot_b + B;
    int4* req = reinterpret_cast<int4*>(wsb + 16 + (size_t)24 * B);
    long long* drow = reinterpret_cast<long long*>(wsb + 16 + (size_t)40 * B);
    auto cu_at = [&](int b) { return derive ? cu[b] + b : cu[b]; };
    const int tid = threadIdx.x;
    const int rounds = (B + NT - 1) / NT;
    const int fc = *a.free_count;

    // pass 1: validate; partial blocks and their refcounts; list the shared ones in order
    int bad = 0, P = 0;
    if (tid == 0 && (cu_at(0) != 0 || cu_at(B) != N)) bad = 1;
    for (int r = 0; r < rounds; ++r) {
        const int b = r * NT + tid;
        int X = -1, r0 = 0;
        if (b < B) {
            const int s = a.seq_lens[b], n = cu_at(b + 1) - cu_at(b);
            if (n < 0 || s < 0 || (long long)s + n > (long long)a.MBR * a.bs) {
                bad = 1;
            } else if (n > 0 && s % a.bs != 0) {
                X = a.tables[(size_t)b * a.MBR + s / a.bs];
                if (X < 0 || X >= a.NB) {
                    bad = 1;
                    X = -1;
                } else {
                    r0 = a.refcount[X];
                }
            }
            req[b] = make_int4(X, r0, 0, 0);
        }
        const int pot = (X >= 0 && r0 > 1) ? 1 : 0;
        int tot;
        const int pos = P + block_excl_scan_i<NT>(pot, redi, &tot);
        if (pot) {
            pot_b[pos] = b;
            pot_X[pos] = X;
        }
        P += tot;
    }
    bad = block_max_i<NT>(bad, redi);
    if (bad) {
        if (tid == 0) {
            ws[0] = 1;
            ws[1] = 0;
            atomicOr(a.state, KV_ERR_APPEND | KV_APPEND_REJECTED);
        }
        return;
    }
    // pass 2: copy-on-write — the i-th sharer (in request order) of block X copies iff
    // i < r0 - 1, which is what processing the batch in order with live refcounts gives;
    // then the pops each request needs, scanned in request order
    int T = 0;
    for (int r = 0; r < rounds; ++r) {
        const int b = r * NT + tid;
        int need = 0;
        int4 q = make_int4(-1, 0, 0, 0);
        if (b < B) {
            const int s = a.seq_lens[b], n = cu_at(b + 1) - cu_at(b);
            q = req[b];
            int cow = 0, conflict = 0;
            if (q.x >= 0 && q.y > 1) {
                int rank = 0, cnt = 0;
                for (int j = 0; j < P; ++j) {
                    if (pot_X[j] == q.x) {
                        ++cnt;
                        if (pot_b[j] < b) ++rank;
                    }
                }
                cow = rank < q.y - 1;
                // another sharer writes X in place in this batch: copy before the scatter
                conflict = cow && cnt > q.y - 1;
            }
            if (n > 0) need = ceil_div(s + n, a.bs) - ceil_div(s, a.bs) + cow;
            q.z = cow | (conflict << 1);
        }
        int tot;
        q.w = T + block_excl_scan_i<NT>(need, redi, &tot);
        T += tot;
        if (b < B) req[b] = q;
    }
    if (T > fc) {
        if (tid == 0) {
            ws[0] = 1;
            atomicOr(a.state, KV_ERR_NOMEM | KV_APPEND_REJECTED);
        }
        return;
    }
    if (tid == 0) {
        ws[1] = 0;
        ws[2] = 0;
    }
    __syncthreads();
    // pass 3: pop, write tables, refcounts, destination rows and lengths
    for (int r = 0; r < rounds; ++r) {
        const int b = r * NT + tid;
        if (b >= B) continue;
        const int s = a.seq_lens[b], n = cu_at(b + 1) - cu_at(b);
        if (n == 0) continue;
        const int4 q = req[b];
        const int cow = q.z & 1, conflict = (q.z >> 1) & 1;
        int p = q.w;
        int* tab = a.tables + (size_t)b * a.MBR;
        if (cow) {
            const int nb = a.free_list[fc - 1 - p++];
            tab[s / a.bs] = nb;
            if ((unsigned)nb < (unsigned)a.NB) {
                a.refcount[nb] = 1;
                atomicSub(&a.refcount[q.x], 1);
                const CowEntry e{q.x, nb, s % a.bs, b};
                if (conflict) list[B - 1 - atomicAdd(&ws[2], 1)] = e;
                else list[atomicAdd(&ws[1], 1)] = e;
            } else {
                atomicOr(a.state, KV_ERR_APPEND);    // corrupt free list
            }
        }
        const int lb_first = ceil_div(s, a.bs);
        const int lb_end = ceil_div(s + n, a.bs);
        for (int lb = lb_first; lb < lb_end; ++lb) {
            const int nb = a.free_list[fc - 1 - p++];
            tab[lb] = nb;
            if ((unsigned)nb < (unsigned)a.NB) a.refcount[nb] = 1;
            else atomicOr(a.state, KV_ERR_APPEND);  // corrupt free list
        }
        // destination rows of the request's new entries, read by the scatter
        const int part_blk = (s % a.bs != 0) ? tab[s / a.bs] : -1;
        const int c0 = cu_at(b);
        for (int t = 0; t < n; ++t) {
            const int pos = s + t;
            const int lb = pos / a.bs;
            const int blk = (lb < lb_first) ? part_blk
                                            : a.free_list[fc - 1 - (q.w + cow + (lb - lb_first))];
            drow[c0 + t] = (unsigned)blk < (unsigned)a.NB ? (long long)blk * a.bs + pos % a.bs : -1;
        }
        a.seq_lens[b] = s + n;
    }
    __syncthreads();
    // copies whose source another request writes in place in this batch happen here,
    // before the scatter starts
    const int nconf = atomicAdd(ws + 2, 0);   // atomics live in L2: read through one
    for (int q = 0; q < nconf; ++q) {
        const CowEntry e = list[B - 1 - q];
        copy_slots(a, e.src, e.dst, e.nslots, tid, NT);
    }
    if (tid == 0) {
        *a.free_count = fc - T;
        ws[0] = 0;
        atomicAnd(a.state, ~KV_APPEND_REJECTED);
    }
}

// Scatter of the new entries: workgroup `wg` of `nwg` handles tokens [tile * tpw, ...) of
// layer / K-V plane lk and moves their rows (H*D bf16, 16-byte pieces) to the destination
// rows the allocation wrote. Thread tid owns piece column tid % lanes of every tpp-th
// token (tpp = nt / lanes tokens per pass when a row has fewer pieces than the group has
// threads), so no per-piece division is needed; P rows per thread are in flight (all
// loads, then all stores). Then the copy-on-write copies, grid-stride over
// (entry, layer, K/V).
template <int P>
SD_DEV void scatter_body(const KvArgs& a, const uint8_t* __restrict__ knew,
                         const uint8_t* __restrict__ vnew, int B, int N, int tpw,
                         const uint8_t* __restrict__ wsb, int tile, int lk, int wg, int nwg,
                         int nt) {
    const int* ws = reinterpret_cast<const int*>(wsb);
    if (ws[0] != 0) return;
    const int tid = threadIdx.x;
    const int l = lk >> 1;
    const size_t ub = (size_t)a.H * a.D * 2;   // bytes of one token's row
    const int lanes = (int)(ub / 16);
    const int tpp = lanes >= nt ? 1 : nt / lanes;            // tokens per pass
    const int rounds = lanes >= nt ? (lanes + nt - 1) / nt : 1;
    const int my_tok = lanes >= nt ? 0 : tid / lanes;
    const int my_q = lanes >= nt ? tid : tid - my_tok * lanes;
    const int t0 = tile * tpw;
    const int ntok = min(tpw, N - t0);
    const int jmax = my_tok < tpp ? (ntok - my_tok + tpp - 1) / tpp : 0;   // tokens of mine
    const long long* drow = reinterpret_cast<const long long*>(wsb + 16 + (size_t)40 * B);
    const uint8_t* src_base = ((lk & 1) ? vnew : knew) + (size_t)l * N * ub;
    uint8_t* dst_base = a.pool + (size_t)lk * a.NB * a.bs * ub;
    for (int j0 = 0; j0 < jmax; j0 += P) {
        long long d[P];
#pragma unroll
        for (int u = 0; u < P; ++u) d[u] = j0 + u < jmax ? drow[t0 + my_tok + (j0 + u) * tpp] : -1;
        for (int r = 0; r < rounds; ++r) {
            const int q = my_q + r * nt;
            if (q >= lanes) break;
            u32x4 v[P];
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int t = t0 + my_tok + (j0 + u) * tpp;
                if (d[u] >= 0)
                    v[u] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(src_base + (size_t)t * ub) + q);
            }
#pragma unroll
            for (int u = 0; u < P; ++u)
                if (d[u] >= 0)
                    __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst_base + (size_t)d[u] * ub) + q);
        }
    }
    const int ncow = ws[1];
    if (ncow > 0) {
        const CowEntry* ce = reinterpret_cast<const CowEntry*>(wsb + 16);
        const size_t per_blk = (size_t)a.bs * ub;
        for (int u = wg; u < ncow * a.L * 2; u += nwg) {
            const CowEntry e = ce[u / (a.L * 2)];
            const int ulk = u % (a.L * 2);
            const uint4* s = reinterpret_cast<const uint4*>(a.pool + ((size_t)ulk * a.NB + e.src) * per_blk);
            uint4* d = reinterpret_cast<uint4*>(a.pool + ((size_t)ulk * a.NB + e.dst) * per_blk);
            const size_t nv = (size_t)e.nslots * ub / 16;
            for (size_t i = tid; i < nv; i += nt) d[i] = s[i];
        }
    }
}

// A tree's accepted path: a nodes, strictly increasing local indices within [0, n).
SD_DEV bool tree_path_ok(const int* __restrict__ path, int a, int n) {
    int prev = -1;
    for (int i = 0; i < a; ++i) {
        const int j = path[i];
        if (j <= prev || j >= n) return false;
        prev = j;
    }
    return true;
}

// Whether request b's tree commit applies: a sound accepted count and path, and the n + 1
// entries of the cycle in the cache.
SD_DEV bool tree_commit_ok(const KvArgs& a, const int* __restrict__ num_acc,
                           const int* __restrict__ nodes, const int* __restrict__ cu, int b,
                           int N) {
    const int lo = cu[b], hi = cu[b + 1], n = hi - lo, acc = num_acc[b], s = a.seq_lens[b];
    return lo >= 0 && hi <= N && n >= 0 && acc >= 0 && acc <= n && s >= n + 1 &&
           (long long)s <= (long long)a.MBR * a.bs && tree_path_ok(nodes + lo, acc, n);
}

// Tree commit, gather: workgroup (b, layer-plane) moves the accepted path's entries of
// request b to the slots after its pending token, in path order (each destination lies
// below every source still to be read; threads keep their 16-byte pieces across copies).
SD_DEV void tree_gather_body(const KvArgs& a, const int* __restrict__ num_acc,
                             const int* __restrict__ nodes, const int* __restrict__ cu, int N,
                             int b, int ulk) {
    if (*a.state & KV_APPEND_REJECTED) return;
    if (!tree_commit_ok(a, num_acc, nodes, cu, b, N)) return;
    const int n = cu[b + 1] - cu[b], acc = num_acc[b];
    const int base = a.seq_lens[b] - (n + 1);
    const size_t ub = (size_t)a.H * a.D * 2;
    const int nvec = (int)(ub / 16);
    for (int i = 1; i <= acc; ++i) {
        const int src = base + 1 + nodes[cu[b] + i - 1], dst = base + i;
        if (src != dst) {
            const int Xs = a.tables[(size_t)b * a.MBR + src / a.bs];
            const int Xd = a.tables[(size_t)b * a.MBR + dst / a.bs];
            if (Xs >= 0 && Xs < a.NB && Xd >= 0 && Xd < a.NB) {
                const u32x4* sp = reinterpret_cast<const u32x4*>(
                    a.pool + (((size_t)ulk * a.NB + Xs) * a.bs + src % a.bs) * ub);
                u32x4* dp = reinterpret_cast<u32x4*>(
                    a.pool + (((size_t)ulk * a.NB + Xd) * a.bs + dst % a.bs) * ub);
                for (int q = threadIdx.x; q < nvec; q += blockDim.x) dp[q] = sp[q];
            }
        }
        __syncthreads();
    }
}

// Rollback of every request by one workgroup of NT threads, for B <= MAXB requests;
// events (freed logical blocks) are processed in windows of EVCAP.
// draft = 1: the draft model's convention, drop max(0, k_b - 1 - a_b) instead of k_b - a_b.
// tree_nodes (tree commit, tree_n nodes): requests whose accepted path or offsets are
// unsound, or that hold fewer than k_b + 1 entries, are skipped and flagged like other
// invalid requests.
template <int NT = kKvNT, int MAXB = SPECDEC_MAX_KV_BATCH, int EVCAP = kEvCap>
SD_DEV void rollback_body(const KvArgs& a, const int* __restrict__ num_acc,
                          const int* __restrict__ cu, int B, int draft = 0,
                          const int* __restrict__ tree_nodes = nullptr, int tree_n = 0) {
    constexpr int RPT = MAXB / NT;    // requests per thread
    constexpr int EPT = EVCAP / NT;   // window events per thread
    static_assert(RPT * NT == MAXB && EPT * NT == EVCAP, "whole rounds per thread");
    __shared__ int redi[NT / kWave];
    __shared__ int s_off[MAXB + 1];
    __shared__ int s_lb0[MAXB];
    __shared__ int s_X[EVCAP];
    __shared__ int s_b[EVCAP];
    __shared__ int s_lb[EVCAP];
    if (*a.state & KV_APPEND_REJECTED) return;
    const int tid = threadIdx.x;
    const int rounds = (B + NT - 1) / NT;
    int fc = *a.free_count;
    int err = 0;
    int newlen[RPT], valid[RPT];
    int E = 0;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int b = i * NT + tid;
        valid[i] = 0;
        newlen[i] = 0;
        int ev = 0;
        if (b < B) {
            const int k = cu[b + 1] - cu[b], acc = num_acc[b], s = a.seq_lens[b];
            const int drop = draft ? max(0, k - 1 - acc) : k - acc;
            if (k < 0 || acc < 0 || acc > k || drop > s ||
                (long long)s > (long long)a.MBR * a.bs ||
                (tree_nodes && !tree_commit_ok(a, num_acc, tree_nodes, cu, b, tree_n))) {
                err = 1;
            } else {
                valid[i] = 1;
                newlen[i] = s - drop;
                ev = ceil_div(s, a.bs) - ceil_div(newlen[i], a.bs);
            }
        }
        if (i < rounds) {
            int tot;
            const int off = E + block_excl_scan_i<NT>(ev, redi, &tot);
            if (b < B) {
                s_off[b] = off;
                s_lb0[b] = ceil_div(newlen[i], a.bs);
            }
            E += tot;
        }
    }
    if (tid == 0) s_off[B] = E;
    __syncthreads();
    for (int w0 = 0; w0 < E; w0 += EVCAP) {
        const int nw = min(EVCAP, E - w0);
        // gather this window's events in (request, logical block) order
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int el = i * NT + tid;
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
        int push[EPT], newrc[EPT], first[EPT];
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int el = i * NT + tid;
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
        int pbase[EPT];
        int ptot = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            int tot;
            pbase[i] = ptot + block_excl_scan_i<NT>(push[i], redi, &tot);
            ptot += tot;
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int el = i * NT + tid;
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
    for (int i = 0; i < RPT; ++i) {
        const int b = i * NT + tid;
        if (b < B && valid[i]) a.seq_lens[b] = newlen[i];
    }
    err = block_max_i<NT>(err, redi);
    if (tid == 0) {
        *a.free_count = min(fc, a.NB);
        if (err) atomicOr(a.state, KV_ERR_ROLLBACK);
    }
}

// ---------------------------------------------------------------------------------------
// Contiguous cache: a buffer per request and a write pointer.
// ---------------------------------------------------------------------------------------
struct ContigArgs {
    uint8_t* pool;
    int L, H, D, max_len, batch;
    int* seq_lens;
    int* state;
};

constexpr int kContigNT = 1024;      // check / commit / rollback workgroup
constexpr int kContigTPW = 16;       // tokens per copy workgroup

// Check of one append (one workgroup): every request's entries fit and the offsets are
// sound; sets or clears KV_APPEND_REJECTED (with KV_ERR_NOMEM / KV_ERR_APPEND).
SD_DEV void contig_check_body(const ContigArgs& a, const int* __restrict__ cu, int B, int N) {
    __shared__ int redi[kContigNT / kWave];
    int nomem = 0, bad = 0;
    for (int b = threadIdx.x; b < B; b += kContigNT) {
        const int n = cu[b + 1] - cu[b], s = a.seq_lens[b];
        if (n < 0 || s < 0 || s > a.max_len) bad = 1;
        else if ((long long)s + n > a.max_len) nomem = 1;
    }
    if (threadIdx.x == 0 && (cu[0] != 0 || cu[B] != N)) bad = 1;
    nomem = block_max_i<kContigNT>(nomem, redi);
    bad = block_max_i<kContigNT>(bad, redi);
    if (threadIdx.x == 0) {
        int st = *a.state & ~KV_APPEND_REJECTED;
        if (bad) st |= KV_ERR_APPEND | KV_APPEND_REJECTED;
        else if (nomem) st |= KV_ERR_NOMEM | KV_APPEND_REJECTED;
        *a.state = st;
    }
}

// Copy of kContigTPW entries of one layer-plane: entry e of request b (cu[b] <= e <
// cu[b+1]) goes to slot seq_lens[b] + (e - cu[b]).
SD_DEV void contig_copy_body(const ContigArgs& a, const uint8_t* __restrict__ knew,
                             const uint8_t* __restrict__ vnew, const int* __restrict__ cu, int B,
                             int N, int tile, int ulk) {
    if (*a.state & KV_APPEND_REJECTED) return;
    const size_t ub = (size_t)a.H * a.D * 2;
    const int nvec = (int)(ub / 16);
    const int l = ulk >> 1, kv = ulk & 1;
    const uint8_t* src = kv ? vnew : knew;
    for (int r = 0; r < kContigTPW; ++r) {
        const int e = tile * kContigTPW + r;
        if (e >= N) break;
        int lo = 0, hi = B;                    // largest b with cu[b] <= e
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu[mid] <= e) lo = mid;
            else hi = mid;
        }
        const int slot = a.seq_lens[lo] + (e - cu[lo]);
        const u32x4* sp = reinterpret_cast<const u32x4*>(src + ((size_t)l * N + e) * ub);
        u32x4* dp = reinterpret_cast<u32x4*>(
            a.pool + ((((size_t)l * 2 + kv) * a.batch + lo) * a.max_len + slot) * ub);
        for (int q = threadIdx.x; q < nvec; q += blockDim.x)
            __builtin_nontemporal_store(__builtin_nontemporal_load(sp + q), dp + q);
    }
}

// Commit of an applied append: the write pointers move past the new entries.
SD_DEV void contig_commit_body(const ContigArgs& a, const int* __restrict__ cu, int B) {
    if (*a.state & KV_APPEND_REJECTED) return;
    for (int b = threadIdx.x; b < B; b += blockDim.x) a.seq_lens[b] += cu[b + 1] - cu[b];
}

// Rewind of every request's write pointer to its committed prefix.
SD_DEV void contig_rollback_body(const ContigArgs& a, const int* __restrict__ num_acc,
                                 const int* __restrict__ cu, int B, int draft) {
    __shared__ int redi[kContigNT / kWave];
    if (*a.state & KV_APPEND_REJECTED) return;
    int err = 0;
    for (int b = threadIdx.x; b < B; b += kContigNT) {
        const int k = cu[b + 1] - cu[b], acc = num_acc[b], s = a.seq_lens[b];
        const int drop = draft ? max(0, k - 1 - acc) : k - acc;
        if (k < 0 || acc < 0 || acc > k || drop > s || s > a.max_len) err = 1;
        else a.seq_lens[b] = s - drop;
    }
    err = block_max_i<kContigNT>(err, redi);
    if (threadIdx.x == 0 && err) atomicOr(a.state, KV_ERR_ROLLBACK);
}

static inline bool contig_ok(const kv_contig_cache* c) {
    if (!c || !c->pool || !c->seq_lens || !c->state) return false;
    if (c->num_layers < 1 || c->num_kv_heads < 1 || c->head_dim < 1 || c->max_len < 1 ||
        c->batch < 1)
        return false;
    if (((size_t)c->num_kv_heads * c->head_dim * 2) % 16 != 0) return false;
    if (((uintptr_t)c->pool & 15) != 0) return false;
    return true;
}

static inline ContigArgs contig_args(const kv_contig_cache* c) {
    ContigArgs a;
    a.pool = reinterpret_cast<uint8_t*>(c->pool);
    a.L = c->num_layers;
    a.H = c->num_kv_heads;
    a.D = c->head_dim;
    a.max_len = c->max_len;
    a.batch = c->batch;
    a.seq_lens = c->seq_lens;
    a.state = c->state;
    return a;
}

static inline bool geometry_ok(const kv_paged_cache* c) {
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

static inline KvArgs args_of(const kv_paged_cache* c) {
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

// Tokens per scatter workgroup for about `ppt` 16-byte pieces per thread.
// Tokens per scatter workgroup of nt threads with ppt rows per thread in flight.
static inline int scatter_tokens_per_wg(const KvArgs& a, int nt, int ppt) {
    const int lanes = (int)((size_t)a.H * a.D * 2 / 16);
    const int tpp = lanes >= nt ? 1 : nt / lanes;
    return tpp * ppt;
}

}  // namespace sd
