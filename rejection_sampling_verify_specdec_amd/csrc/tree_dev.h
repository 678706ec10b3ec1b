// Verification of a draft tree by a team of workgroups per request (gfx950).
//
// The rule generalizes "Speculative decoding: accelerate LLM generation without changing
// its answers", section 2, to several proposals for the same position: the children of a
// node are tried in node order, each accepted with probability min(1, p'(y) / q(y)) where
// p' starts as the node's target distribution p and, after each rejected child, becomes
// the normalized residual normalize(max(0, p' - q)) (the same residual as at a linear
// rejection; section 3's argument applied at each rejection keeps the output distributed
// as p). The first accepted child continues the walk; when all are rejected the
// replacement is drawn from the last residual; a node reached by acceptance without
// children yields the bonus token from its p. The accepted path is what "Keep cache
// validity aligned with the committed token history", paragraph 3, has the cache keep.
//
// The walk is sequential per request and reads only the rows it visits: one pass over a
// position's target (and draft) row for its max and exp-sum, one pass over the row pair
// per rejected child (its residual mass, summed per 2048-token sub-chunk), and a rescan of
// one sub-chunk for the draw. The passes themselves are split among the team (see
// "Teams" below); every member takes the same decisions from the same combined sums.

#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "verify_dev.h"

namespace sd {

constexpr int kTreeNT = 1024;                    // threads of a walk workgroup
constexpr int kTreeTile = kTreeNT * 8;           // tokens per tile, 8 consecutive per thread
constexpr int kTreeSub = 2048;                   // tokens per sub-chunk (256 threads)
constexpr int kTreeMaxSub = SPECDEC_MAX_V / kTreeSub;
static_assert(kTreeMaxSub <= kTreeNT, "one sub-chunk sum per thread in the draw");
static_assert(SPECDEC_MAX_TREE <= kWave, "a wave ballot covers the nodes of a request");

struct TreeArgs {
    const uint8_t* tgt;      // [N+B][V] target rows by position
    const uint8_t* dft;      // [N+B][V] draft rows by position (leaves not read)
    const int* tokens;       // [N]
    const int* parent;       // [N] -1 or an earlier node of the request
    const int* cu;           // [B+1]
    const float* u_acc;      // [N] the uniform of each node's accept test
    const float* u_smp;      // [B]
    int B, N, max_nodes, V;
    float c;                 // log2(e) / T
    int* out_tokens;         // [N+B]
    int* nodes_out;          // [N] accepted path per request, from cu[b]
    int* num_acc;            // [B]
    int* num_emit;           // [B]
    int* err_word;           // [1]
    int* req_flags;          // [B] or null
    double* ring;            // [(N + 2B) * slot]: request b's passes from (cu[b] + 2b) * slot
    int* ctr;                // [B * kTreeCtrStride]: ticket and done counters, zeroed first
    int nchunk;              // chunks (two tiles) per pass
    int nsub;                // sub-chunks of a row
    int slot;                // doubles per pass: 64 * nchunk (4 per wave and chunk)
    int team;                // workgroups per request
    int spin_limit;          // polls a member waits for the others before it gives up
    // top-k / top-p: every row's threshold and its kept tokens' max and exp-sum, from the
    // select launches (target row r at r, draft row r at rows + r); null with temperature
    // alone, where the walk takes each position's statistics itself
    const float* thr;
    const RowPartial* part;
    int rows;                // N + B
    // bf16 with top-k / top-p: each target row's kept tokens listed in ascending order
    // ([N+B] counts, -1 when not listed; [N+B][kKeptCap] tokens and their keys), else null
    const int* kn;
    const uint32_t* ktok;
    const uint16_t* kkey;
    // per-request transforms: every row's parameters ([N+B] target rows, then draft rows),
    // the request's log2(e) / T read from its root row; null with scalars
    const RowParams* rpar;
};

// Eight consecutive tokens of a row kept as loaded (bf16 stays packed: 4 VGPRs); tokens at
// or past V read as -inf.
template <bool BF16>
struct Tok8 {
    u32x4 v[BF16 ? 1 : 2];
    SD_DEV float get(int e) const {
        if constexpr (BF16) {
            const uint32_t w = v[0][e >> 1];
            return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
        } else {
            return __uint_as_float(v[e >> 2][e & 3]);
        }
    }
};

template <bool BF16, bool VEC>
SD_DEV Tok8<BF16> load8r(const uint8_t* __restrict__ row, int V, int i0) {
    Tok8<BF16> t;
    constexpr uint32_t NINF = BF16 ? 0xff80ff80u : 0xff800000u;
    if constexpr (VEC) {
        // whole 16-byte vectors: V * size is a multiple of 16, so i0 < V covers all 8
        const u32x4* p = reinterpret_cast<const u32x4*>(row) + (BF16 ? i0 / 8 : i0 / 4);
#pragma unroll
        for (int h = 0; h < (BF16 ? 1 : 2); ++h)
            t.v[h] = i0 < V ? __builtin_nontemporal_load(p + h) : (u32x4){NINF, NINF, NINF, NINF};
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t bits;
            if constexpr (BF16)
                bits = i0 + e < V ? (uint32_t)reinterpret_cast<const uint16_t*>(row)[i0 + e] : 0xff80u;
            else
                bits = i0 + e < V ? reinterpret_cast<const uint32_t*>(row)[i0 + e] : NINF;
            if constexpr (BF16) {
                if (e & 1) t.v[0][e >> 1] |= bits << 16;
                else t.v[0][e >> 1] = bits;
            } else {
                t.v[e >> 2][e & 3] = bits;
            }
        }
    }
    return t;
}

// A position's two rows as the walk weighs them: p(x) = exp2(z c - mct) * alt for a target
// logit z >= tt, 0 below it; q(x) likewise from the draft row (tt = td = -inf without top-k
// or top-p).
struct RowNorm {
    float mct, mcd, tt, td;
    double alt, ald;
};

// The exponential form of the linear path: p(x) = exp2(z c - mc) * al, 0 for z = -inf or
// below the row's threshold.
SD_DEV double tree_prob(float z, float c, float mc, double al, float thr) {
    return (z > -INFINITY && z >= thr) ? (double)__builtin_amdgcn_exp2f(fmaf(z, c, -mc)) * al
                                       : 0.0;
}

// Residual chain: f_0 = p, f_{s+1} = max(0, f_s - q) / W_s, with Winv[s] = 1 / W_s.
SD_DEV double tree_chain(double p, double q, const double* Winv, int t) {
    double f = p;
    for (int s = 0; s < t; ++s) f = fmax(f - q, 0.0) * Winv[s];
    return f;
}

enum : int { TW_P = 0, TW_RESID = 1, TW_TESTED = 2 };

// Weight of a token for the draw or the residual mass: TW_P p (bonus), TW_RESID
// max(0, f_{t-1} - q) (the residual after t rejections, unnormalized), TW_TESTED f_t.
SD_DEV double tree_weight(float zt, float zd, int kind, int t, float c, const RowNorm& r,
                          const double* W) {
    const double p = tree_prob(zt, c, r.mct, r.alt, r.tt);
    if (kind == TW_P) return p;
    const double q = tree_prob(zd, c, r.mcd, r.ald, r.td);
    if (kind == TW_TESTED) return tree_chain(p, q, W, t);
    return fmax(tree_chain(p, q, W, t - 1) - q, 0.0);
}

// ---------------------------------------------------------------------------------------
// Teams: G workgroups share one request's walk. Every pass over a position's rows is cut
// into chunks of two tiles (16384 tokens, 8 sub-chunks); a workgroup takes the next chunk
// with an atomic ticket, writes the chunk's per-sub-chunk partials to the request's slot
// of the workspace ring and counts the chunk done. Every member then waits for the whole
// pass, combines the partials in a fixed order and takes the same decisions, so the
// results do not depend on G or on which member computed which chunk. Tickets are only
// waited for once a running workgroup holds them, so the wait always ends; it is bounded
// all the same (SPECDEC_ERR_TEAM). A request makes at most n + 2 passes (one stats pass
// per visited position, one per rejected child, one for the final draw), each with its
// own slot, so a member that starts late replays the walk from the ring.
// ---------------------------------------------------------------------------------------

constexpr int kTreeChunk = 2 * kTreeTile;                 // tokens per ticket
constexpr int kTreeSubPerChunk = kTreeChunk / kTreeSub;   // 8
constexpr int kTreeMaxTeam = 16;
constexpr int kTreeCtrStride = 64;                        // ints per request: claim, done
constexpr int kTreeDoneOff = 32;                          // done on its own 128-byte line
constexpr int kTreeSpinLimit = 1 << 20;
enum : int { TK_STATS = 3 };                              // pass kinds besides TW_*

struct TeamLds {
    int tk[2];                          // this workgroup's ticket, double-buffered
    int timeout;
};

// The ring and the counters are shared by workgroups on different XCDs, whose L2 caches
// are not coherent with each other. Every ring access is an agent-scope atomic, and the
// pass is published by release / acquire at agent scope: the waves' ring stores precede
// the workgroup barrier, after which one thread adds the member's chunks to the done count
// with release order; the waiting thread polls the count with relaxed loads, then issues
// an agent-scope acquire fence before the barrier that lets its workgroup read the ring.
// Happens-before thus runs writer waves -> barrier -> release -> acquire -> barrier ->
// reader waves, each link at a scope that holds both ends. (On gfx950 the release writes
// back and the acquire invalidates the XCD's L2: measured 8% of the walk at 128 requests.)
// A team of one (solo) shares nothing: plain stores and loads, ordered by the workgroup
// barrier.
SD_DEV void ring_put(double* p, double x, bool solo) {
    if (solo) *p = x;
    else __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
SD_DEV double ring_get(const double* p, bool solo) {
    if (solo) return *p;
    return __hip_atomic_load(const_cast<double*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Max m and S = sum exp2(z c - fl(m c)) of two tiles of one row over this wave (1024
// tokens), m NaN when they hold NaN / +inf (every lane gets the wave's values).
template <class T8>
SD_DEV void wave_stats2(const T8& za, const T8& zb, float c, double* m_out, double* s_out) {
    float z[16];
    float tm = -INFINITY;
    int bad = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        z[e] = za.get(e);
        z[8 + e] = zb.get(e);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        bad |= (z[e] != z[e]) | (z[e] == INFINITY);
        tm = fmaxf(tm, z[e]);
    }
    const float m = wave_max(tm);
    float acc = 0.f;
    if (m > -INFINITY) {
        const float mc = m * c;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += __builtin_amdgcn_exp2f(fmaf(z[e], c, -mc));
    }
    *m_out = wave_max_i(bad) ? (double)NAN : (double)m;
    *s_out = wave_sum((double)acc);
}

// Weight of a token in a pass (tree_weight without the -inf tests: exp2 of -inf is 0, and
// -inf >= -inf holds).
SD_DEV double team_prob(float z, float c, float mc, double al, float thr) {
    return z >= thr ? (double)__builtin_amdgcn_exp2f(fmaf(z, c, -mc)) * al : 0.0;
}
SD_DEV double team_weight(float zt, float zd, int kind, int t, float c, const RowNorm& r,
                          const double* W) {
    const double p = team_prob(zt, c, r.mct, r.alt, r.tt);
    if (kind == TW_P) return p;
    const double q = team_prob(zd, c, r.mcd, r.ald, r.td);
    if (kind == TW_TESTED) return tree_chain(p, q, W, t);
    return fmax(tree_chain(p, q, W, t - 1) - q, 0.0);
}

constexpr int kTreeWaveSpan = kTreeChunk / (kTreeNT / kWave);   // 1024 tokens per wave
static_assert(kTreeSub == 2 * kTreeWaveSpan, "a sub-chunk is two waves' spans");

// A chunk of the target row and, with DR, of the draft row: its loads.
template <bool BF16>
struct Quad {
    Tok8<BF16> t0, t1, d0, d1;
};

// Eight tokens at i0 < V from whole 16-byte vectors (no bounds test).
template <bool BF16>
SD_DEV Tok8<BF16> load8f(const uint8_t* __restrict__ row, int i0) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + (BF16 ? i0 / 8 : i0 / 4);
    Tok8<BF16> t;
#pragma unroll
    for (int h = 0; h < (BF16 ? 1 : 2); ++h) t.v[h] = __builtin_nontemporal_load(p + h);
    return t;
}

// FULL: the chunk lies inside the row and rows are whole vectors, so every load is issued
// unconditionally (the compiler can then keep the next chunk's loads in flight).
// Wave w of the workgroup covers the chunk's tokens [w * 1024, w * 1024 + 1024): lane l
// takes 8 at l * 8 and 8 at 512 + l * 8 (each load instruction reads 1 KB contiguous).
template <bool BF16, bool VEC, bool DR, bool FULL>
SD_DEV Quad<BF16> team_load(const TreeArgs& a, const uint8_t* trow, const uint8_t* drow, int ch) {
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    const int i0 = ch * kTreeChunk + w * kTreeWaveSpan + l * 8, i1 = i0 + kTreeWaveSpan / 2;
    Quad<BF16> q;
    if constexpr (FULL && VEC) {
        q.t0 = load8f<BF16>(trow, i0);
        q.t1 = load8f<BF16>(trow, i1);
        if constexpr (DR) {
            q.d0 = load8f<BF16>(drow, i0);
            q.d1 = load8f<BF16>(drow, i1);
        }
    } else {
        q.t0 = load8r<BF16, VEC>(trow, a.V, i0);
        q.t1 = load8r<BF16, VEC>(trow, a.V, i1);
        if constexpr (DR) {
            q.d0 = load8r<BF16, VEC>(drow, a.V, i0);
            q.d1 = load8r<BF16, VEC>(drow, a.V, i1);
        }
    }
    return q;
}

// Pass kinds as compile-time cases of the chunk loop.
enum : int { KC_STATS = 0, KC_P = 1, KC_RESID1 = 2, KC_CHAIN = 3 };

// One chunk of a pass: every wave writes the partials of its 1024 tokens (entry wc =
// chunk * 16 + wave) to the slot. Stats: slot[4 wc ..] = (m_t, s_t, m_d, s_d); weights:
// slot[wc] = the wave's sum (sub-chunk q, 2048 tokens, is entries 2q and 2q + 1).
template <bool BF16, int KC>
SD_DEV void team_compute(const TreeArgs& a, const Quad<BF16>& q, int ch, int kind, bool both,
                         int t, const RowNorm& r, const double* W, double* slot) {
    const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
    const int wc = ch * (kTreeNT / kWave) + w;
    const bool solo = a.team == 1;
    if constexpr (KC == KC_STATS) {
        double m, sm;
        wave_stats2(q.t0, q.t1, a.c, &m, &sm);
        if (l == 0) {
            ring_put(slot + 4 * wc, m, solo);
            ring_put(slot + 4 * wc + 1, sm, solo);
        }
        if (both) {
            wave_stats2(q.d0, q.d1, a.c, &m, &sm);
            if (l == 0) {
                ring_put(slot + 4 * wc + 2, m, solo);
                ring_put(slot + 4 * wc + 3, sm, solo);
            }
        }
    } else {
        double s0 = 0.0, s1 = 0.0;
        if constexpr (KC == KC_P) {              // the bonus: p alone
#pragma unroll
            for (int e = 0; e < 8; ++e) s0 += team_prob(q.t0.get(e), a.c, r.mct, r.alt, r.tt);
#pragma unroll
            for (int e = 0; e < 8; ++e) s1 += team_prob(q.t1.get(e), a.c, r.mct, r.alt, r.tt);
        } else if constexpr (KC == KC_RESID1) {  // the first residual, max(0, p - q)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                s0 += fmax(team_prob(q.t0.get(e), a.c, r.mct, r.alt, r.tt) -
                           team_prob(q.d0.get(e), a.c, r.mcd, r.ald, r.td), 0.0);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                s1 += fmax(team_prob(q.t1.get(e), a.c, r.mct, r.alt, r.tt) -
                           team_prob(q.d1.get(e), a.c, r.mcd, r.ald, r.td), 0.0);
        } else {                                 // longer residual chains, tested weights
#pragma unroll 2
            for (int e = 0; e < 8; ++e) {
                s0 += team_weight(q.t0.get(e), q.d0.get(e), kind, t, a.c, r, W);
                s1 += team_weight(q.t1.get(e), q.d1.get(e), kind, t, a.c, r, W);
            }
        }
        const double sw = wave_sum(s0 + s1);
        if (l == 0) ring_put(slot + wc, sw, solo);
    }
}

// Chunks [c0, c1) of a pass: whole chunks with the next one's loads in flight (except for
// the register-hungry chains), then a chunk that reaches past the row end with
// bounds-tested loads.
template <bool BF16, bool VEC, bool DR, int KC>
SD_DEV void team_slice(const TreeArgs& a, const uint8_t* trow, const uint8_t* drow, int c0,
                       int c1, int kind, bool both, int t, const RowNorm& r, const double* W,
                       double* slot) {
    constexpr bool PIPE = KC != KC_CHAIN;
    const int cfull = VEC ? min(c1, a.V / kTreeChunk) : c0;
    if (c0 < cfull) {
        if constexpr (PIPE) {
            Quad<BF16> cur = team_load<BF16, VEC, DR, true>(a, trow, drow, c0);
            for (int ch = c0; ch + 1 < cfull; ++ch) {
                const Quad<BF16> nxt = team_load<BF16, VEC, DR, true>(a, trow, drow, ch + 1);
                team_compute<BF16, KC>(a, cur, ch, kind, both, t, r, W, slot);
                cur = nxt;
            }
            team_compute<BF16, KC>(a, cur, cfull - 1, kind, both, t, r, W, slot);
        } else {
            for (int ch = c0; ch < cfull; ++ch) {
                const Quad<BF16> q = team_load<BF16, VEC, DR, true>(a, trow, drow, ch);
                team_compute<BF16, KC>(a, q, ch, kind, both, t, r, W, slot);
            }
        }
    }
    for (int ch = max(c0, cfull); ch < c1; ++ch) {
        const Quad<BF16> q = team_load<BF16, VEC, DR, false>(a, trow, drow, ch);
        team_compute<BF16, KC>(a, q, ch, kind, both, t, r, W, slot);
    }
}

// Pass k of request b by this member. A ticket is a slice of ceil(C / G) chunks (pass k:
// tickets [k NS, (k + 1) NS), NS slices); the member takes slices while its ticket lies in
// pass k (a ticket past it is kept for a later pass), counts its chunks done once its
// stores have completed, then waits until all C chunks of the pass are done. `par` picks
// the half of tk[] holding the current ticket. Returns false when the wait ran past its
// bound.
template <bool BF16, bool VEC>
SD_DEV bool team_pass(const TreeArgs& a, const uint8_t* trow, const uint8_t* drow, int k,
                      int kind, bool both, int t, const RowNorm& r, const double* W, double* slot,
                      int* claim, int* done, TeamLds& s, int& par) {
    const int tid = threadIdx.x, l = tid % kWave;
    const int C = a.nchunk, S = (C + a.team - 1) / a.team, NS = (C + S - 1) / S;
    const bool solo = a.team == 1;
    int mine = 0;                                     // chunks this member finished
    for (;;) {
        const int tk = solo ? k : s.tk[par];          // solo: the whole pass, no tickets
        if (tk >= (k + 1) * NS) break;
        int nx = 0;
        if (tid == 0 && !solo)
            nx = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int c0 = (tk - k * NS) * S, c1 = min(C, c0 + S);
        if (kind == TK_STATS) {
            if (both)
                team_slice<BF16, VEC, true, KC_STATS>(a, trow, drow, c0, c1, kind, both, t, r, W,
                                                      slot);
            else
                team_slice<BF16, VEC, false, KC_STATS>(a, trow, drow, c0, c1, kind, both, t, r, W,
                                                       slot);
        } else if (kind == TW_P) {
            team_slice<BF16, VEC, false, KC_P>(a, trow, drow, c0, c1, kind, both, t, r, W, slot);
        } else if (kind == TW_RESID && t == 1) {
            team_slice<BF16, VEC, true, KC_RESID1>(a, trow, drow, c0, c1, kind, both, t, r, W,
                                                   slot);
        } else {
            team_slice<BF16, VEC, true, KC_CHAIN>(a, trow, drow, c0, c1, kind, both, t, r, W, slot);
        }
        mine += c1 - c0;
        if (solo) break;
        // the other half: its last readers passed the barrier below one slice ago
        if (tid == 0) s.tk[par ^ 1] = nx;
        par ^= 1;
        __syncthreads();
    }
    if (solo) {
        __syncthreads();                              // the partials are visible to the WG
        return true;
    }
    __syncthreads();
    if (tid == 0) {
        if (mine) __hip_atomic_fetch_add(done, mine, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        int it = 0, to = 0;
        while (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (k + 1) * C) {
            if (++it > a.spin_limit) {
                to = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s.timeout = to;
    }
    __syncthreads();
    return s.timeout == 0;
}

// Workgroup max / sum of two values at once, each in the order block_max / block_sum use
// (lane butterfly, then waves in index order). red2 holds 2 * NT / 64 entries.
SD_DEV void block_max2(float& x, float& y, float* red2) {
    x = wave_max(x);
    y = wave_max(y);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    constexpr int NW = kTreeNT / kWave;
    if (l == 0) { red2[w] = x; red2[NW + w] = y; }
    __syncthreads();
    x = red2[0];
    y = red2[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) { x = fmaxf(x, red2[i]); y = fmaxf(y, red2[NW + i]); }
    __syncthreads();
}
SD_DEV void block_sum2(double& x, double& y, double* red2) {
    x = wave_sum(x);
    y = wave_sum(y);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    constexpr int NW = kTreeNT / kWave;
    if (l == 0) { red2[w] = x; red2[NW + w] = y; }
    __syncthreads();
    x = red2[0];
    y = red2[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) { x += red2[i]; y += red2[NW + i]; }
    __syncthreads();
}

// Max and S = sum exp2((z - m) c) of the target row and (with both) the draft row from a
// stats slot: entries wc = 0 .. 16 C - 1 combined in index order (thread i takes i and
// i + 1024); S is NaN when the row holds NaN / +inf.
SD_DEV void team_stats_final(const TreeArgs& a, const double* slot, bool both, float* mt,
                             double* St, float* md, double* Sd, double* red2, float* redf2,
                             int* redi) {
    const int tid = threadIdx.x;
    const bool solo = a.team == 1;
    const int nwc = a.nchunk * (kTreeNT / kWave);
    // this thread's entries (at most two), each row's (m, s)
    double m_[2][2], s_[2][2];
    int bad = 0;
    float mx_t = -INFINITY, mx_d = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = tid + h * kTreeNT;
        m_[h][0] = m_[h][1] = -INFINITY;
        s_[h][0] = s_[h][1] = 0.0;
        if (i < nwc) {
            m_[h][0] = ring_get(slot + 4 * i, solo);
            s_[h][0] = ring_get(slot + 4 * i + 1, solo);
            if (both) {
                m_[h][1] = ring_get(slot + 4 * i + 2, solo);
                s_[h][1] = ring_get(slot + 4 * i + 3, solo);
            }
        }
        bad |= (m_[h][0] != m_[h][0]) | ((m_[h][1] != m_[h][1]) << 1);
        mx_t = fmaxf(mx_t, (float)m_[h][0]);
        mx_d = fmaxf(mx_d, (float)m_[h][1]);
    }
    bad = block_max_i<kTreeNT>(bad, redi);
    block_max2(mx_t, mx_d, redf2);
    const float mct = mx_t * a.c, mcd = mx_d * a.c;
    double xt = 0.0, xd = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (m_[h][0] > -INFINITY) xt += s_[h][0] * exp2((double)((float)m_[h][0] * a.c) - (double)mct);
        if (m_[h][1] > -INFINITY) xd += s_[h][1] * exp2((double)((float)m_[h][1] * a.c) - (double)mcd);
    }
    block_sum2(xt, xd, red2);
    *mt = mx_t;
    *md = mx_d;
    *St = (bad & 1) ? (double)NAN : (mx_t > -INFINITY ? xt * exp2(-(double)fmaf(mx_t, a.c, -mct)) : 0.0);
    *Sd = (bad & 2) ? (double)NAN : (mx_d > -INFINITY ? xd * exp2(-(double)fmaf(mx_d, a.c, -mcd)) : 0.0);
}

// Sub-chunk q's weight sum: its two waves' entries in order.
SD_DEV double team_weight_sub(const double* slot, int q, bool solo) {
    return ring_get(slot + 2 * q, solo) + ring_get(slot + 2 * q + 1, solo);
}

// The total of a weight slot, sub-chunks in index order.
SD_DEV double team_weight_total(const TreeArgs& a, const double* slot, double* red) {
    const int tid = threadIdx.x;
    return block_sum<kTreeNT>(tid < a.nsub ? team_weight_sub(slot, tid, a.team == 1) : 0.0, red);
}

// Inverse CDF over the weights whose sub-chunk sums are in sub[]: the smallest x with
// C(x) > u * W (ascending ids, W the total of the sub-chunk sums in scan order), or the
// last x with positive weight if rounding leaves none.
template <bool BF16, bool VEC>
SD_DEV int tree_draw(const TreeArgs& a, const uint8_t* trow, const uint8_t* drow, int kind,
                     int t, const RowNorm& r, const double* W, const double* sub, float u,
                     double* red, int* redi) {
    const int tid = threadIdx.x;
    const int nsub = (a.V + kTreeSub - 1) / kTreeSub;
    // the sub-chunk holding t: exclusive prefix of the sub-chunk sums, fixed order
    const double mysub = tid < nsub ? sub[tid] : 0.0;
    double tot;
    const double before = block_excl_scan_d<kTreeNT>(mysub, red, &tot);
    const double tt = (double)u * tot;
    int cand = (tid < nsub && before + mysub > tt && mysub > 0.0) ? tid : 0x7fffffff;
    int s = block_min_i<kTreeNT>(cand, redi);
    bool last = false;
    if (s == 0x7fffffff) {                       // rounding: the last positive sub-chunk
        s = block_max_i<kTreeNT>(tid < nsub && mysub > 0.0 ? tid : -1, redi);
        last = true;
        if (s < 0) return -1;
    }
    double base = 0.0;
    if (tid == s) red[kTreeNT / kWave] = before;
    __syncthreads();
    base = red[kTreeNT / kWave];
    __syncthreads();
    // rescan the sub-chunk: 256 threads x 8 tokens
    const int i0 = s * kTreeSub + tid * 8;
    double wv[8];
    double run = 0.0;
    if (tid < kTreeSub / 8) {
        float zt[8], zd[8];
        load8<BF16, VEC>(trow, a.V, i0, zt);
        if (kind != TW_P) load8<BF16, VEC>(drow, a.V, i0, zd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            wv[e] = tree_weight(zt[e], kind != TW_P ? zd[e] : -INFINITY, kind, t, a.c, r, W);
            run += wv[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = 0.0;
    }
    double stot;
    double C = base + block_excl_scan_d<kTreeNT>(run, red, &stot);
    int mine = 0x7fffffff, lastpos = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (tid >= kTreeSub / 8 || i0 + e >= a.V) continue;
        C += wv[e];
        if (mine == 0x7fffffff && C > tt && wv[e] > 0.0) mine = i0 + e;
        if (wv[e] > 0.0) lastpos = i0 + e;
    }
    int x = last ? 0x7fffffff : block_min_i<kTreeNT>(mine, redi);
    if (x == 0x7fffffff) x = block_max_i<kTreeNT>(lastpos, redi);
    return x;
}

// A target row whose kept tokens are listed: every weight off the list is 0 (p = 0 there),
// so a pass is a sum over at most kKeptCap entries, which each member of a team takes by
// itself (same entries, same order, same result) with no ring and no wait. Thread i takes
// entry i; *tok is its token (-1 past the list).
static_assert(kKeptCap <= kTreeNT, "one listed token per thread");
SD_DEV double listed_weight(const TreeArgs& a, int rt, const uint8_t* drow, int nl, int kind,
                            int t, const RowNorm& r, const double* W, int* tok) {
    const int i = threadIdx.x;
    *tok = -1;
    if (i >= nl) return 0.0;
    const int x = (int)a.ktok[(size_t)rt * kKeptCap + i];
    const float zt = key_to_float<true>(a.kkey[(size_t)rt * kKeptCap + i]);
    const float zd = kind != TW_P ? load_elem(drow, x, true) : -INFINITY;
    *tok = x;
    return tree_weight(zt, zd, kind, t, a.c, r, W);
}

// Inverse CDF over a listed row (ascending ids): the smallest listed x with C(x) > u * W,
// or the last with positive weight if rounding leaves none; -1 when nothing has weight.
SD_DEV int listed_draw(const TreeArgs& a, int rt, const uint8_t* drow, int nl, int kind, int t,
                       const RowNorm& r, const double* W, float u, double* red, int* redi) {
    int x;
    const double w = listed_weight(a, rt, drow, nl, kind, t, r, W, &x);
    double tot;
    const double C = block_excl_scan_d<kTreeNT>(w, red, &tot);
    const double tt = (double)u * tot;
    const bool pos = x >= 0 && w > 0.0;
    int i = block_min_i<kTreeNT>(pos && C + w > tt ? (int)threadIdx.x : 0x7fffffff, redi);
    if (i == 0x7fffffff) i = block_max_i<kTreeNT>(pos ? (int)threadIdx.x : -1, redi);
    return i < 0 ? -1 : (int)a.ktok[(size_t)rt * kKeptCap + i];
}

// The walk of request b by member `mem` of its team; member 0 draws and writes the outputs.
template <bool BF16, bool VEC>
SD_DEV void tree_walk_body(const TreeArgs& args, int b, int mem) {
    TreeArgs a = args;           // with per-request transforms a.c becomes the request's own
    using Lt = Layout<BF16, VEC>;
    __shared__ double red[kTreeNT / kWave + 1];
    __shared__ int redi[kTreeNT / kWave];
    __shared__ double sub[kTreeMaxSub];
    __shared__ double sW[SPECDEC_MAX_TREE];        // 1 / W_s of the residuals so far
    __shared__ int s_path[SPECDEC_MAX_TREE];
    __shared__ float s_zt[SPECDEC_MAX_TREE], s_zd[SPECDEC_MAX_TREE];
    __shared__ int s_flags;
    __shared__ unsigned long long s_kids;
    __shared__ int s_next;
    __shared__ TeamLds tl;
    __shared__ double red2[2 * (kTreeNT / kWave)];
    __shared__ float redf2[2 * (kTreeNT / kWave)];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int lo = a.cu[b], hi = a.cu[b + 1], n = hi - lo;
    const bool bad_k = a.cu[0] != 0 || a.cu[a.B] != a.N || n < 0 || n > a.max_nodes || lo < 0 ||
                       hi > a.N;
    if (bad_k) {
        if (tid == 0 && mem == 0) {
            a.num_acc[b] = -1;
            a.num_emit[b] = 0;
            atomicOr(a.err_word, SPECDEC_ERR_K);
            if (a.req_flags) a.req_flags[b] = SPECDEC_ERR_K;
        }
        return;
    }
    const bool bad_param = a.rpar && (a.rpar[lo + b].flags & kRpBad);
    if (a.rpar) a.c = a.rpar[lo + b].c;
    // validity of the tree, its tokens, uniforms and parameters (wave 0, a lane per node)
    if (tid < kWave) {
        int f = 0;
        if (lane < n) {
            const int pa = a.parent[lo + lane], y = a.tokens[lo + lane];
            const float u = a.u_acc[lo + lane];
            if (pa < -1 || pa >= lane) f |= SPECDEC_ERR_TREE;
            if (y < 0 || y >= a.V) f |= SPECDEC_ERR_TOKEN;
            if (!(u >= 0.0f && u < 1.0f)) f |= SPECDEC_ERR_UNIFORM;
        }
        if (lane == 0) {
            const float us = a.u_smp[b];
            if (!(us >= 0.0f && us < 1.0f)) f |= SPECDEC_ERR_UNIFORM;
            if (bad_param) f |= SPECDEC_ERR_PARAM;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, kWave);
        if (lane == 0) s_flags = f;
    }
    __syncthreads();
    int flags = s_flags;
    int na = 0, x = -1;
    if (!flags) {
        int* claim = a.ctr + (size_t)b * kTreeCtrStride;
        int* done = claim + kTreeDoneOff;
        double* ring = a.ring + (size_t)(lo + 2 * b) * a.slot;
        if (tid == 0 && a.team > 1)
            tl.tk[0] = __hip_atomic_fetch_add(claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        int par = 0;                                 // tl.tk[par]: the current ticket
        int k = 0;      // passes so far: at most n + 2 (ring slots), checked before each
        int wslot = -1, kind = TW_RESID, t = 0;      // the final draw's slot, kind, residual
        bool ldraw = false;                          // the final draw is over a listed row
        int nl = -1, rt = 0;                         // the position's listed tokens, its row
        RowNorm rn{0.f, 0.f, -INFINITY, -INFINITY, 0.0, 0.0};
        const RowNorm none{0.f, 0.f, -INFINITY, -INFINITY, 0.0, 0.0};
        const uint8_t* trow = nullptr;
        const uint8_t* drow = nullptr;
        int v = 0;                                   // position: 0 root, 1 + j node j
        while (true) {
            trow = a.tgt + (size_t)(lo + b + v) * a.V * Lt::ES;
            drow = a.dft + (size_t)(lo + b + v) * a.V * Lt::ES;
            if (tid < kWave) {
                const bool kid = lane < n && a.parent[lo + lane] == v - 1;
                const unsigned long long m = __ballot(kid);
                if (lane == 0) s_kids = m;
                // the children's logits at this position, for their accept tests (the
                // loads complete during the stats pass)
                if (kid) {
                    const int y = a.tokens[lo + lane];
                    s_zt[lane] = load_elem(trow, y, BF16);
                    s_zd[lane] = load_elem(drow, y, BF16);
                }
            }
            __syncthreads();
            unsigned long long kids = s_kids;
            float mt, md = 0.f;
            double St, Sd = 1.0;
            rt = lo + b + v;
            if (a.part) {
                // top-k / top-p: the select launches' statistics of the kept tokens
                const RowPartial pt = a.part[rt];
                mt = pt.m;
                St = pt.s;
                rn.tt = a.thr[rt];
                if (kids) {
                    const RowPartial pd = a.part[a.rows + rt];
                    md = pd.m;
                    Sd = pd.s;
                    rn.td = a.thr[a.rows + rt];
                }
            } else {
                if (k > n + 1 ||
                    !team_pass<BF16, VEC>(a, trow, drow, k, TK_STATS, kids != 0, 0, none, sW,
                                          ring + (size_t)k * a.slot, claim, done, tl, par)) {
                    flags |= SPECDEC_ERR_TEAM;
                    break;
                }
                team_stats_final(a, ring + (size_t)k * a.slot, kids != 0, &mt, &St, &md, &Sd,
                                 red2, redf2, redi);
                if (!kids) {
                    md = 0.f;
                    Sd = 1.0;
                }
                ++k;
            }
            if (!(St > 0.0 && St < INFINITY && mt > -INFINITY) ||
                (kids && !(Sd > 0.0 && Sd < INFINITY && md > -INFINITY))) {
                flags |= SPECDEC_ERR_NONFINITE;
                break;
            }
            nl = a.kn ? a.kn[rt] : -1;
            rn.mct = mt * a.c;
            rn.mcd = md * a.c;
            rn.alt = exp2(-(double)fmaf(mt, a.c, -rn.mct)) / St;
            rn.ald = kids ? exp2(-(double)fmaf(md, a.c, -rn.mcd)) / Sd : 0.0;
            if (!kids && nl >= 0) {                  // bonus from a listed p
                ldraw = true;
                kind = TW_P;
                t = 0;
                break;
            }
            if (!kids) {                             // bonus from p at a leaf
                if (k > n + 1 ||
                    !team_pass<BF16, VEC>(a, trow, drow, k, TW_P, false, 0, rn, sW,
                                          ring + (size_t)k * a.slot, claim, done, tl, par)) {
                    flags |= SPECDEC_ERR_TEAM;
                    break;
                }
                wslot = k++;
                ldraw = false;
                kind = TW_P;
                t = 0;
                break;
            }
            t = 0;
            kind = TW_RESID;
            int next = -1;
            while (kids) {
                const int j = __ffsll((long long)kids) - 1;
                kids &= kids - 1;
                if (tid == 0) {
                    const float zt = s_zt[j], zd = s_zd[j];
                    const double q = tree_prob(zd, a.c, rn.mcd, rn.ald, rn.td);
                    const double P = tree_chain(tree_prob(zt, a.c, rn.mct, rn.alt, rn.tt), q, sW, t);
                    if (q == 0.0) s_flags |= SPECDEC_ERR_QZERO;
                    s_next = ((double)a.u_acc[lo + j] * q < P) ? j : -1;
                }
                __syncthreads();
                next = s_next;
                __syncthreads();
                if (next >= 0) break;
                // rejected: the residual mass after t + 1 rejections
                double Wn;
                if (nl >= 0) {
                    int x_;
                    Wn = block_sum<kTreeNT>(
                        listed_weight(a, rt, drow, nl, TW_RESID, t + 1, rn, sW, &x_), red);
                    ldraw = true;
                } else {
                    if (k > n + 1 ||
                        !team_pass<BF16, VEC>(a, trow, drow, k, TW_RESID, true, t + 1, rn, sW,
                                              ring + (size_t)k * a.slot, claim, done, tl, par)) {
                        flags |= SPECDEC_ERR_TEAM;
                        break;
                    }
                    Wn = team_weight_total(a, ring + (size_t)k * a.slot, red);
                    wslot = k++;
                    ldraw = false;
                }
                if (!(Wn > kResidFloor)) {
                    // no residual mass (not possible in exact arithmetic): draw from the
                    // distribution the child was tested against
                    flags |= SPECDEC_ERR_ZFALLBACK;
                    kind = TW_TESTED;
                    if (ldraw) break;
                    if (k > n + 1 ||
                        !team_pass<BF16, VEC>(a, trow, drow, k, TW_TESTED, true, t, rn, sW,
                                              ring + (size_t)k * a.slot, claim, done, tl, par)) {
                        flags |= SPECDEC_ERR_TEAM;
                        break;
                    }
                    wslot = k++;
                    break;
                }
                if (tid == 0) sW[t] = 1.0 / Wn;
                __syncthreads();
                ++t;
            }
            if (flags & SPECDEC_ERR_TEAM) break;
            if (next >= 0) {
                if (tid == 0) s_path[na] = next;
                ++na;
                v = next + 1;
                continue;
            }
            break;                                   // every child rejected
        }
        // the replacement (from the last residual, or the tested distribution after a zero
        // residual) or the bonus: member 0 rescans one sub-chunk
        if (mem == 0 && ldraw && !(flags & (SPECDEC_ERR_NONFINITE | SPECDEC_ERR_TEAM))) {
            x = listed_draw(a, rt, drow, nl, kind, t, rn, sW, a.u_smp[b], red, redi);
        } else if (mem == 0 && wslot >= 0 &&
                   !(flags & (SPECDEC_ERR_NONFINITE | SPECDEC_ERR_TEAM))) {
            const double* sl = ring + (size_t)wslot * a.slot;
            for (int q = tid; q < a.nsub; q += kTreeNT) sub[q] = team_weight_sub(sl, q, a.team == 1);
            __syncthreads();
            x = tree_draw<BF16, VEC>(a, trow, drow, kind, t, rn, sW, sub,
                                     a.u_smp[b], red, redi);
        }
        __syncthreads();
        flags |= s_flags;
    }
    if (mem != 0) return;
    if (x < 0 && !(flags & (SPECDEC_ERR_TOKEN | SPECDEC_ERR_UNIFORM | SPECDEC_ERR_TREE |
                            SPECDEC_ERR_TEAM | SPECDEC_ERR_PARAM)))
        flags |= SPECDEC_ERR_NONFINITE;          // nothing to draw from
    const bool err = (flags & (SPECDEC_ERR_TOKEN | SPECDEC_ERR_UNIFORM | SPECDEC_ERR_NONFINITE |
                               SPECDEC_ERR_TREE | SPECDEC_ERR_TEAM | SPECDEC_ERR_PARAM)) != 0;
    if (tid < na && !err) {
        a.nodes_out[lo + tid] = s_path[tid];
        a.out_tokens[lo + b + tid] = a.tokens[lo + s_path[tid]];
    }
    if (tid == 0) {
        if (!err) a.out_tokens[lo + b + na] = x;
        a.num_acc[b] = err ? -1 : na;
        a.num_emit[b] = err ? 0 : na + 1;
        if (flags) atomicOr(a.err_word, flags);
        if (a.req_flags) a.req_flags[b] = flags;
    }
}

}  // namespace sd
