// Verification of a draft tree, one workgroup per request (gfx950).
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
// one sub-chunk for the draw. A workgroup of 1024 threads keeps 64 KB of loads in flight.

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
constexpr int kTreeSubPerTile = kTreeTile / kTreeSub;
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

// The exponential form of the linear path: p(x) = exp2(z c - mc) * al, 0 for z = -inf.
SD_DEV double tree_prob(float z, float c, float mc, double al) {
    return z > -INFINITY ? (double)__builtin_amdgcn_exp2f(fmaf(z, c, -mc)) * al : 0.0;
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
SD_DEV double tree_weight(float zt, float zd, int kind, int t, float c, float mct, double alt,
                          float mcd, double ald, const double* W) {
    const double p = tree_prob(zt, c, mct, alt);
    if (kind == TW_P) return p;
    const double q = tree_prob(zd, c, mcd, ald);
    if (kind == TW_TESTED) return tree_chain(p, q, W, t);
    return fmax(tree_chain(p, q, W, t - 1) - q, 0.0);
}

// Running max / exp-sum of one thread's share of a row: the sum is kept in units of
// exp2(z c - fl(m c)) and rescaled when the max grows.
struct RowAcc {
    float m = -INFINITY;
    double s = 0.0;
    int bad = 0;
    template <class T8>
    SD_DEV void add(const T8& z8, float c) {
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = z8.get(e);
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bad |= (z[e] != z[e]) | (z[e] == INFINITY);
            mt = fmaxf(mt, z[e]);
        }
        if (mt > m) {
            if (m > -INFINITY) s *= exp2((double)(m * c) - (double)(mt * c));
            m = mt;
        }
        if (m > -INFINITY) {
            const float mc = m * c;
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += __builtin_amdgcn_exp2f(fmaf(z[e], c, -mc));
            s += (double)acc;
        }
    }
};

// Workgroup max and S = sum exp2((z - m) c) from the threads' accumulators (fixed order);
// NaN when the row holds NaN / +inf.
SD_DEV double row_acc_finish(const RowAcc& r, float c, float* m_out, double* red, float* redf,
                             int* redi) {
    const int bad = block_max_i<kTreeNT>(r.bad, redi);
    const float m = block_max<kTreeNT>(r.m, redf);
    const float mc = m * c;
    const double mine = r.m > -INFINITY ? r.s * exp2((double)(r.m * c) - (double)mc) : 0.0;
    const double S = block_sum<kTreeNT>(mine, red);
    *m_out = m;
    if (bad) return (double)NAN;
    // from units of exp2(z c - mc) to exp2((z - m) c): m c = mc + emc exactly
    return m > -INFINITY ? S * exp2(-(double)fmaf(m, c, -mc)) : 0.0;
}

// Max and exp-sum of a position's target row and, with both, of its draft row, in one
// pass with two tiles of loads in flight per thread.
template <bool BF16, bool VEC>
SD_DEV void tree_row_stats(const uint8_t* trow, const uint8_t* drow, bool both, int V, float c,
                           float* mt, double* St, float* md, double* Sd, double* red,
                           float* redf, int* redi) {
    const int tid = threadIdx.x;
    RowAcc at, ad;
    for (int i0 = tid * 8; i0 < V; i0 += 2 * kTreeTile) {
        const int i1 = i0 + kTreeTile;
        const Tok8<BF16> z0 = load8r<BF16, VEC>(trow, V, i0), z1 = load8r<BF16, VEC>(trow, V, i1);
        Tok8<BF16> y0, y1;
        if (both) {
            y0 = load8r<BF16, VEC>(drow, V, i0);
            y1 = load8r<BF16, VEC>(drow, V, i1);
        }
        at.add(z0, c);
        at.add(z1, c);
        if (both) {
            ad.add(y0, c);
            ad.add(y1, c);
        }
    }
    *St = row_acc_finish(at, c, mt, red, redf, redi);
    if (both) *Sd = row_acc_finish(ad, c, md, red, redf, redi);
}

// One pass over the row pair with two tiles of loads in flight per thread: sub-chunk sums
// of the weights into sub[] (LDS; every wave's sum of a tile goes to wsub, then four wave
// sums per sub-chunk, fixed order); returns the total (fixed order).
constexpr int kTreeMaxTile = SPECDEC_MAX_V / kTreeTile;
template <bool BF16, bool VEC>
SD_DEV double tree_pass(const TreeArgs& a, const uint8_t* trow, const uint8_t* drow, int kind,
                        int t, float mct, double alt, float mcd, double ald, const double* W,
                        double* sub, double* wsub, double* red) {
    constexpr int NW = kTreeNT / kWave;
    const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
    const int ntile = (a.V + kTreeTile - 1) / kTreeTile;
    for (int tile = 0; tile < ntile; tile += 2) {
        const int i0 = tile * kTreeTile + tid * 8, i1 = i0 + kTreeTile;
        const Tok8<BF16> zt0 = load8r<BF16, VEC>(trow, a.V, i0);
        const Tok8<BF16> zt1 = load8r<BF16, VEC>(trow, a.V, i1);
        Tok8<BF16> zd0, zd1;
        if (kind != TW_P) {
            zd0 = load8r<BF16, VEC>(drow, a.V, i0);
            zd1 = load8r<BF16, VEC>(drow, a.V, i1);
        }
        double s0 = 0.0, s1 = 0.0;
#pragma unroll 2
        for (int e = 0; e < 8; ++e) {
            s0 += tree_weight(zt0.get(e), kind != TW_P ? zd0.get(e) : -INFINITY, kind, t, a.c,
                              mct, alt, mcd, ald, W);
            s1 += tree_weight(zt1.get(e), kind != TW_P ? zd1.get(e) : -INFINITY, kind, t, a.c,
                              mct, alt, mcd, ald, W);
        }
        s0 = wave_sum(s0);
        s1 = wave_sum(s1);
        if (l == 0) {
            wsub[tile * NW + w] = s0;
            if (tile + 1 < ntile) wsub[(tile + 1) * NW + w] = s1;
        }
    }
    __syncthreads();
    constexpr int WPS = kTreeSub / 8 / kWave;          // waves per sub-chunk
    for (int q = tid; q < ntile * kTreeSubPerTile; q += kTreeNT) {
        double x = 0.0;
#pragma unroll
        for (int i = 0; i < WPS; ++i) x += wsub[q * WPS + i];
        sub[q] = x;
    }
    __syncthreads();
    // the total, in a fixed order (sub-chunks past the vocabulary hold 0)
    const int nsub = (a.V + kTreeSub - 1) / kTreeSub;
    return block_sum<kTreeNT>(tid < nsub ? sub[tid] : 0.0, red);
}

// Inverse CDF over the weights whose sub-chunk sums are in sub[]: the smallest x with
// C(x) > u * W (ascending ids, W the total of the sub-chunk sums in scan order), or the
// last x with positive weight if rounding leaves none.
template <bool BF16, bool VEC>
SD_DEV int tree_draw(const TreeArgs& a, const uint8_t* trow, const uint8_t* drow, int kind,
                     int t, float mct, double alt, float mcd, double ald, const double* W,
                     const double* sub, float u, double* red, int* redi) {
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
            wv[e] = tree_weight(zt[e], kind != TW_P ? zd[e] : -INFINITY, kind, t, a.c, mct, alt,
                                mcd, ald, W);
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

// The walk of request b.
template <bool BF16, bool VEC>
SD_DEV void tree_walk_body(const TreeArgs& a, int b) {
    using Lt = Layout<BF16, VEC>;
    __shared__ double red[kTreeNT / kWave + 1];
    __shared__ double wsub[kTreeMaxTile * (kTreeNT / kWave)];
    __shared__ float redf[kTreeNT / kWave];
    __shared__ int redi[kTreeNT / kWave];
    __shared__ double sub[kTreeMaxSub];
    __shared__ double sW[SPECDEC_MAX_TREE];        // 1 / W_s of the residuals so far
    __shared__ int s_path[SPECDEC_MAX_TREE];
    __shared__ int s_flags, s_x;
    __shared__ unsigned long long s_kids;
    __shared__ int s_next;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int lo = a.cu[b], hi = a.cu[b + 1], n = hi - lo;
    const bool bad_k = a.cu[0] != 0 || a.cu[a.B] != a.N || n < 0 || n > a.max_nodes || lo < 0 ||
                       hi > a.N;
    if (bad_k) {
        if (tid == 0) {
            a.num_acc[b] = -1;
            a.num_emit[b] = 0;
            atomicOr(a.err_word, SPECDEC_ERR_K);
            if (a.req_flags) a.req_flags[b] = SPECDEC_ERR_K;
        }
        return;
    }
    // validity of the tree, its tokens and uniforms (wave 0, a lane per node)
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
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, kWave);
        if (lane == 0) s_flags = f;
    }
    __syncthreads();
    int flags = s_flags;
    int na = 0, x = -1;
    if (!flags) {
        int v = 0;                                   // position: 0 root, 1 + j node j
        while (true) {
            const uint8_t* trow = a.tgt + (size_t)(lo + b + v) * a.V * Lt::ES;
            const uint8_t* drow = a.dft + (size_t)(lo + b + v) * a.V * Lt::ES;
            if (tid < kWave) {
                const bool kid = lane < n && a.parent[lo + lane] == v - 1;
                const unsigned long long m = __ballot(kid);
                if (lane == 0) s_kids = m;
            }
            __syncthreads();
            unsigned long long kids = s_kids;
            float mt, md = 0.f;
            double St, Sd = 1.0;
            tree_row_stats<BF16, VEC>(trow, drow, kids != 0, a.V, a.c, &mt, &St, &md, &Sd, red,
                                      redf, redi);
            if (!(St > 0.0 && St < INFINITY && mt > -INFINITY) ||
                (kids && !(Sd > 0.0 && Sd < INFINITY && md > -INFINITY))) {
                flags |= SPECDEC_ERR_NONFINITE;
                break;
            }
            const float mct = mt * a.c, mcd = md * a.c;
            const double alt = exp2(-(double)fmaf(mt, a.c, -mct)) / St;
            const double ald = kids ? exp2(-(double)fmaf(md, a.c, -mcd)) / Sd : 0.0;
            if (!kids) {                             // bonus from p at a leaf
                const double Wt = tree_pass<BF16, VEC>(a, trow, drow, TW_P, 0, mct, alt, mcd,
                                                       ald, sW, sub, wsub, red);
                (void)Wt;
                x = tree_draw<BF16, VEC>(a, trow, drow, TW_P, 0, mct, alt, mcd, ald, sW, sub,
                                         a.u_smp[b], red, redi);
                break;
            }
            int t = 0, kind = TW_RESID;
            int next = -1;
            while (kids) {
                const int j = __ffsll((long long)kids) - 1;
                kids &= kids - 1;
                if (tid == 0) {
                    const int y = a.tokens[lo + j];
                    const float zt = load_elem(trow, y, BF16), zd = load_elem(drow, y, BF16);
                    const double q = tree_prob(zd, a.c, mcd, ald);
                    const double P = tree_chain(tree_prob(zt, a.c, mct, alt), q, sW, t);
                    if (q == 0.0) s_flags |= SPECDEC_ERR_QZERO;
                    s_next = ((double)a.u_acc[lo + j] * q < P) ? j : -1;
                }
                __syncthreads();
                next = s_next;
                __syncthreads();
                if (next >= 0) break;
                // rejected: the residual mass after t + 1 rejections
                const double Wn = tree_pass<BF16, VEC>(a, trow, drow, TW_RESID, t + 1, mct, alt,
                                                       mcd, ald, sW, sub, wsub, red);
                if (!(Wn > 0.0)) {
                    // no residual mass (not possible in exact arithmetic): draw from the
                    // distribution the child was tested against
                    flags |= SPECDEC_ERR_ZFALLBACK;
                    kind = TW_TESTED;
                    (void)tree_pass<BF16, VEC>(a, trow, drow, TW_TESTED, t, mct, alt, mcd, ald, sW,
                                               sub, wsub, red);
                    break;
                }
                if (tid == 0) sW[t] = 1.0 / Wn;
                __syncthreads();
                ++t;
            }
            if (next >= 0) {
                if (tid == 0) s_path[na] = next;
                ++na;
                v = next + 1;
                continue;
            }
            // every child rejected: the replacement from the last residual (or the tested
            // distribution after a zero residual)
            x = tree_draw<BF16, VEC>(a, trow, drow, kind, t, mct, alt, mcd, ald, sW, sub,
                                     a.u_smp[b], red, redi);
            break;
        }
        __syncthreads();
        flags |= s_flags;
    }
    if (x < 0 && !(flags & (SPECDEC_ERR_TOKEN | SPECDEC_ERR_UNIFORM | SPECDEC_ERR_TREE)))
        flags |= SPECDEC_ERR_NONFINITE;          // nothing to draw from
    const bool err = (flags & (SPECDEC_ERR_TOKEN | SPECDEC_ERR_UNIFORM | SPECDEC_ERR_NONFINITE |
                               SPECDEC_ERR_TREE)) != 0;
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
