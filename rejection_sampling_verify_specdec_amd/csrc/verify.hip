// Batched speculative-decoding verification for gfx950 (MI355X).
//
// What is computed follows "Speculative decoding: accelerate LLM generation without
// changing its answers", section 2 "Draft, verify, correct" (accept y_i with probability
// min(1, p_i(y_i)/q_i(y_i)) left to right, replacement from normalize(max(0, p_j - q_j))
// at the first rejection j, bonus token from p_{k+1} when all are accepted), with the
// decoding transform (temperature, top-k) applied identically to target and draft rows
// and a max-subtracted (stable) softmax (same page, section 6).
//
// Pipeline on one stream, per call:
//   k_row_stats   every target and draft row is streamed once in 16 KB-32 KB chunks with
//                 128-bit loads; each workgroup writes the chunk max m_c and
//                 S_c = sum exp2((z - m_c) * c), c = log2(e) / T, as an fp32/fp64 pair.
//   k_topk_rows   (top-k only) one workgroup per row: exact top-k threshold, max and
//                 kept-set sum (replaces k_row_stats).
//   k_decide      one wave per request: combines the row partials in fp64, evaluates
//                 p_i(y_i), q_i(y_i) in fp64, the accept test u * q < p, finds the first
//                 rejection, writes accepted tokens and the parameters of the one row
//                 pair (or bonus row) still to be sampled.
//   k_resid_part  per (request, chunk): partial sums of the sampling weights w(x) =
//                 max(0, p_j(x) - q_j(x)) (or p_{k+1}(x) for the bonus), fp64.
//   k_resid_pick  per request: total W, t = u * W, locates the chunk holding t, then an
//                 LDS prefix scan over that chunk in ascending token order finds the
//                 smallest x with C(x) > t. Rows after the first rejection are never
//                 re-read (ragged early exit).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "specdec.h"

namespace sd {

constexpr int kNT = 256;        // threads per workgroup of the streaming kernels
constexpr int kVPT = 8;         // 16-byte vectors per thread per chunk
constexpr int kTopkNT = 1024;   // threads per workgroup of the top-k row kernel

enum : int { MODE_NONE = 0, MODE_RESID = 1, MODE_BONUS = 2 };

// Partial statistics of one row chunk (or of a whole row for top-k rows).
struct alignas(16) RowPartial {
    float m;      // max logit of the chunk (-inf if none)
    int nkept;    // kept tokens (top-k rows only)
    double s;     // sum over the chunk of exp2((z - m) * c)
};

// What k_decide leaves for the sampling kernels, per request.
struct alignas(16) SampleRec {
    int mode, row_t, row_d, out_pos;
    float mc_t, mc_d;      // fp32(m * c): the exponent offset used elementwise
    float thr_t, thr_d;    // top-k thresholds (-inf when off)
    double al_t, al_d;     // 2^(m*c - mc) / S: turns exp2(z*c - mc) into a probability
    float u;
    int flags;
    int pad0, pad1;
};

template <bool BF16, bool VEC>
struct Layout {
    static constexpr int ES = BF16 ? 2 : 4;          // element bytes
    static constexpr int EPV = 16 / ES;              // elements per 16-byte vector
    static constexpr int PER = VEC ? EPV : 1;        // elements per thread per column
    static constexpr int COLS = VEC ? kVPT : kVPT * EPV;
    static constexpr int EPT = COLS * PER;           // elements per thread per chunk
    static constexpr int CH = kNT * EPT;             // elements per chunk
};

SD_DEV float load_elem(const uint8_t* row, long i, bool bf16) {
    if (bf16) return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(row)[i]) << 16);
    return reinterpret_cast<const float*>(row)[i];
}

// Element z[col * PER + e] of the calling thread is index c0 + (col * kNT + tid) * PER + e
// of the row; elements at or past V read as -inf.
template <bool BF16, bool VEC>
SD_DEV void load_chunk(const uint8_t* __restrict__ row, int V, int c0,
                       float (&z)[Layout<BF16, VEC>::EPT]) {
    using Lt = Layout<BF16, VEC>;
    const int tid = threadIdx.x;
    if constexpr (VEC) {
        const uint4* p = reinterpret_cast<const uint4*>(row);
        uint4 raw[Lt::COLS];
#pragma unroll
        for (int col = 0; col < Lt::COLS; ++col) {
            const int i0 = c0 + (col * kNT + tid) * Lt::PER;
            if (i0 < V) {
                raw[col] = p[i0 / Lt::EPV];
            } else {
                raw[col] = BF16 ? make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u)
                                : make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
            }
        }
#pragma unroll
        for (int col = 0; col < Lt::COLS; ++col) {
            const uint32_t w[4] = {raw[col].x, raw[col].y, raw[col].z, raw[col].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (BF16) {
                    z[col * Lt::PER + 2 * q] = bf16_lo(w[q]);
                    z[col * Lt::PER + 2 * q + 1] = bf16_hi(w[q]);
                } else {
                    z[col * Lt::PER + q] = __uint_as_float(w[q]);
                }
            }
        }
    } else {
#pragma unroll
        for (int col = 0; col < Lt::COLS; ++col) {
            const int i = c0 + col * kNT + tid;
            z[col] = i < V ? load_elem(row, i, BF16) : -INFINITY;
        }
    }
}

template <int N>
SD_DEV float tree_sum(float (&a)[N]) {
#pragma unroll
    for (int s = 1; s < N; s <<= 1) {
#pragma unroll
        for (int i = 0; i + s < N; i += 2 * s) a[i] += a[i + s];
    }
    return a[0];
}

SD_DEV const uint8_t* row_ptr(const uint8_t* tgt, const uint8_t* dft, int rows_t, int row,
                              int V, int es) {
    return row < rows_t ? tgt + (size_t)row * V * es : dft + (size_t)(row - rows_t) * V * es;
}

// ---------------------------------------------------------------------------------------
// Row statistics, chunked: max and sum of exp2((z - m_c) * c) per chunk.
// ---------------------------------------------------------------------------------------
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_row_stats(const uint8_t* __restrict__ tgt,
                                                   const uint8_t* __restrict__ dft,
                                                   int rows_t, int V, int nchunks, float c,
                                                   RowPartial* __restrict__ part) {
    using Lt = Layout<BF16, VEC>;
    __shared__ float redf[kNT / kWave];
    __shared__ double redd[kNT / kWave];
    __shared__ int redi[kNT / kWave];
    const int row = blockIdx.x / nchunks;
    const int chunk = blockIdx.x - row * nchunks;
    const uint8_t* base = row_ptr(tgt, dft, rows_t, row, V, Lt::ES);
    float z[Lt::EPT];
    load_chunk<BF16, VEC>(base, V, chunk * Lt::CH, z);

    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < Lt::EPT; ++i) mx = fmaxf(mx, z[i]);
    const float m = block_max<kNT>(mx, redf);

    double s;
    if (m == -INFINITY) {
        // nothing finite: the chunk contributes 0, unless it holds a NaN
        int nan = 0;
#pragma unroll
        for (int i = 0; i < Lt::EPT; ++i) nan |= (z[i] != z[i]);
        nan = block_max_i<kNT>(nan, redi);
        s = nan ? (double)NAN : 0.0;
    } else {
        const float mc = m * c;
        const float emc = fmaf(m, c, -mc);    // exact: m * c = mc + emc
        float vs[Lt::COLS];
#pragma unroll
        for (int col = 0; col < Lt::COLS; ++col) {
            float e[Lt::PER];
#pragma unroll
            for (int q = 0; q < Lt::PER; ++q)
                e[q] = __builtin_amdgcn_exp2f(fmaf(z[col * Lt::PER + q], c, -mc));
            vs[col] = tree_sum(e);
        }
        const double tot = block_sum<kNT>((double)tree_sum(vs), redd);
        // exp2(z*c - mc) = exp2((z - m)*c) * 2^emc, so rescale by 2^-emc
        s = tot * exp2(-(double)emc);
    }
    if (threadIdx.x == 0) {
        RowPartial rp;
        rp.m = m;
        rp.nkept = 0;
        rp.s = s;
        part[blockIdx.x] = rp;
    }
}

// ---------------------------------------------------------------------------------------
// Top-k rows: one workgroup of 1024 threads per row. The row is walked in segments of
// 1024 * 8 vectors. Exact k-th largest value by a 4-pass radix select on
// order-preserving 32-bit keys (2 passes suffice for bf16, whose low 16 key bits are
// constant), then kept-set max / count / sum in a final pass.
// ---------------------------------------------------------------------------------------
SD_DEV uint32_t f2key(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
SD_DEV float key2f(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kTopkNT) void k_topk_rows(const uint8_t* __restrict__ tgt,
                                                       const uint8_t* __restrict__ dft,
                                                       int rows_t, int V, int top_k, float c,
                                                       RowPartial* __restrict__ part,
                                                       float* __restrict__ row_thr) {
    constexpr int NT = kTopkNT;
    constexpr int ES = BF16 ? 2 : 4;
    __shared__ unsigned hist[256];
    __shared__ float redf[NT / kWave];
    __shared__ double redd[NT / kWave];
    __shared__ int redi[NT / kWave];
    __shared__ uint32_t s_prefix;
    __shared__ int s_krem;
    const int row = blockIdx.x;
    const uint8_t* base = row_ptr(tgt, dft, rows_t, row, V, ES);
    const int tid = threadIdx.x;

    // pass 0: max, invalid entries (NaN, +inf)
    float mx = -INFINITY;
    int bad = 0;
    for (int i = tid; i < V; i += NT) {
        const float z = load_elem(base, i, BF16);
        mx = fmaxf(mx, z);
        bad |= (z != z) | (z == INFINITY);
    }
    const float m = block_max<NT>(mx, redf);
    bad = block_max_i<NT>(bad, redi);

    // radix select of the top_k-th largest key
    if (tid == 0) {
        s_prefix = 0;
        s_krem = top_k;
    }
    __syncthreads();
    const int npass = BF16 ? 2 : 4;
    for (int pass = 0; pass < npass; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        const uint32_t prefix = s_prefix;
        const uint32_t hmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
        for (int i = tid; i < V; i += NT) {
            const uint32_t k = f2key(load_elem(base, i, BF16));
            if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & 0xff], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            int krem = s_krem;
            int d = 255;
            for (; d > 0; --d) {
                if ((int)hist[d] >= krem) break;
                krem -= hist[d];
            }
            s_prefix = prefix | ((uint32_t)d << shift);
            s_krem = krem;
        }
        __syncthreads();
    }
    uint32_t tkey = s_prefix;
    if (BF16) tkey |= (tkey & 0x80000000u) ? 0u : 0xffffu;   // negatives' low key bits are 1s
    const float thr = key2f(tkey);

    // kept set: z >= thr (and finite); max is the row max; count and sum
    const float mc = m * c;
    const float emc = fmaf(m, c, -mc);
    float acc = 0.f;
    int cnt = 0;
    for (int i = tid; i < V; i += NT) {
        const float z = load_elem(base, i, BF16);
        if (z >= thr && z > -INFINITY) {
            acc += __builtin_amdgcn_exp2f(fmaf(z, c, -mc));
            ++cnt;
        }
    }
    const double tot = block_sum<NT>((double)acc, redd);
    cnt = block_sum_i<NT>(cnt, redi);
    if (tid == 0) {
        RowPartial rp;
        rp.m = m;
        rp.nkept = cnt;
        rp.s = bad ? (double)NAN : (m == -INFINITY ? 0.0 : tot * exp2(-(double)emc));
        part[row] = rp;
        row_thr[row] = thr;
    }
}

// ---------------------------------------------------------------------------------------
// Per-request decision: one wave per request.
// ---------------------------------------------------------------------------------------
struct DecideArgs {
    const uint8_t* tgt;
    const uint8_t* dft;
    int bf16;
    const int* tokens;
    const int* cu;
    const float* u_acc;
    const float* u_smp;
    int B, K, max_k, V;
    int nparts;              // partials per row
    int topk;                // 1 when rows carry a top-k threshold
    float c;
    const RowPartial* part;
    const float* row_thr;
    int* out_tokens;
    int* num_acc;
    int* num_emit;
    int* err_word;
    SampleRec* rec;
    specdec_debug dbg;
};

__global__ __launch_bounds__(kWave) void k_decide(DecideArgs a) {
    __shared__ float s_m[2 * SPECDEC_MAX_K + 1];
    __shared__ double s_S[2 * SPECDEC_MAX_K + 1];
    __shared__ float s_thr[2 * SPECDEC_MAX_K + 1];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int rows_t = a.K + a.B;
    const int lo = a.cu[b], hi = a.cu[b + 1];
    const int k = hi - lo;
    const bool bad_k = a.cu[0] != 0 || a.cu[a.B] != a.K || k < 0 || k > a.max_k || lo < 0 ||
                       hi > a.K;
    if (bad_k) {
        if (lane == 0) {
            a.num_acc[b] = -1;
            a.num_emit[b] = 0;
            a.rec[b].mode = MODE_NONE;
            atomicOr(a.err_word, SPECDEC_ERR_K);
            if (a.dbg.req_flags) a.dbg.req_flags[b] = SPECDEC_ERR_K;
        }
        return;
    }
    const double cd = (double)a.c;
    const int nrows = 2 * k + 1;
    int row_bad = 0;
    for (int r = lane; r < nrows; r += kWave) {
        const int prow = r <= k ? lo + b + r : rows_t + lo + (r - k - 1);
        const RowPartial* pp = a.part + (size_t)prow * a.nparts;
        float m = -INFINITY;
        for (int q = 0; q < a.nparts; ++q) m = fmaxf(m, pp[q].m);
        double S = 0.0;
        int nk = 0;
        for (int q = 0; q < a.nparts; ++q) {
            const RowPartial x = pp[q];
            // chunks with no finite entry carry 0 (or NaN, which must propagate)
            S += x.m == -INFINITY ? x.s : x.s * exp2((double)(x.m - m) * cd);
            nk += x.nkept;
        }
        const float thr = a.topk ? a.row_thr[prow] : -INFINITY;
        s_m[r] = m;
        s_S[r] = S;
        s_thr[r] = thr;
        row_bad |= !(S > 0.0 && S < INFINITY && m > -INFINITY);
        if (a.dbg.row_max) a.dbg.row_max[prow] = m;
        if (a.dbg.row_sum) a.dbg.row_sum[prow] = S;
        if (a.dbg.row_thr) a.dbg.row_thr[prow] = thr;
        if (a.dbg.row_nkept) a.dbg.row_nkept[prow] = a.topk ? nk : -1;
    }
    __syncthreads();

    // proposals: lane i handles position i (k <= SPECDEC_MAX_K = kWave)
    int flags = 0;
    bool acc = true;
    double P = 0.0, Q = 0.0;
    int y = 0;
    if (lane < k) {
        y = a.tokens[lo + lane];
        const double u = (double)a.u_acc[lo + lane];
        if (!(u >= 0.0 && u < 1.0)) flags |= SPECDEC_ERR_UNIFORM;
        if (y < 0 || y >= a.V) {
            flags |= SPECDEC_ERR_TOKEN;
        } else {
            const int es = a.bf16 ? 2 : 4;
            const float zt = load_elem(a.tgt + (size_t)(lo + b + lane) * a.V * es, y, a.bf16);
            const float zd = load_elem(a.dft + (size_t)(lo + lane) * a.V * es, y, a.bf16);
            const int rt = lane, rd = k + 1 + lane;
            if (zt >= s_thr[rt] && zt > -INFINITY)
                P = exp2(((double)zt - (double)s_m[rt]) * cd) / s_S[rt];
            if (zd >= s_thr[rd] && zd > -INFINITY)
                Q = exp2(((double)zd - (double)s_m[rd]) * cd) / s_S[rd];
            acc = u * Q < P;
        }
    }
    const double us = (double)a.u_smp[b];
    if (lane == 0 && !(us >= 0.0 && us < 1.0)) flags |= SPECDEC_ERR_UNIFORM;
    if (row_bad) flags |= SPECDEC_ERR_NONFINITE;
    const unsigned long long rej = __ballot(lane < k && !acc);
    const int j = rej ? (__ffsll((long long)rej) - 1) : k;
    if (lane < k && lane <= j && Q == 0.0 && !(flags & SPECDEC_ERR_TOKEN)) flags |= SPECDEC_ERR_QZERO;
    // OR the flags over the wave
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) flags |= __shfl_xor(flags, o, kWave);

    if (lane < k) {
        if (a.dbg.p_y) a.dbg.p_y[lo + lane] = P;
        if (a.dbg.q_y) a.dbg.q_y[lo + lane] = Q;
    }
    const bool err = (flags & (SPECDEC_ERR_TOKEN | SPECDEC_ERR_UNIFORM | SPECDEC_ERR_NONFINITE)) != 0;
    if (err) {
        if (lane == 0) {
            a.num_acc[b] = -1;
            a.num_emit[b] = 0;
            a.rec[b].mode = MODE_NONE;
            atomicOr(a.err_word, flags);
            if (a.dbg.req_flags) a.dbg.req_flags[b] = flags;
        }
        return;
    }
    if (lane < j) a.out_tokens[lo + b + lane] = y;
    if (lane == 0) {
        a.num_acc[b] = j;
        a.num_emit[b] = j + 1;
        SampleRec r;
        r.mode = j < k ? MODE_RESID : MODE_BONUS;
        r.row_t = lo + b + j;
        r.row_d = j < k ? lo + j : 0;
        r.out_pos = lo + b + j;
        const float mt = s_m[j];
        r.mc_t = mt * a.c;
        r.al_t = exp2(-(double)fmaf(mt, a.c, -r.mc_t)) / s_S[j];
        r.thr_t = s_thr[j];
        if (j < k) {
            const float md = s_m[k + 1 + j];
            r.mc_d = md * a.c;
            r.al_d = exp2(-(double)fmaf(md, a.c, -r.mc_d)) / s_S[k + 1 + j];
            r.thr_d = s_thr[k + 1 + j];
        } else {
            r.mc_d = 0.f;
            r.al_d = 0.0;
            r.thr_d = INFINITY;
        }
        r.u = a.u_smp[b];
        r.flags = flags;
        r.pad0 = r.pad1 = 0;
        a.rec[b] = r;
        if (flags) atomicOr(a.err_word, flags);
        if (a.dbg.req_flags) a.dbg.req_flags[b] = flags;
    }
}

// ---------------------------------------------------------------------------------------
// Sampling weights and the inverse CDF.
// ---------------------------------------------------------------------------------------
// w(x) = max(0, p(x) - q(x)) for a replacement, p(x) for the bonus; p and q in fp64 from
// fp32 exponentials of the same form the statistics used.
SD_DEV double weight(float zt, float zd, const SampleRec& r, float c, bool resid) {
    const double pt = zt >= r.thr_t
                          ? (double)__builtin_amdgcn_exp2f(fmaf(zt, c, -r.mc_t)) * r.al_t
                          : 0.0;
    if (!resid) return pt;
    const double pd = zd >= r.thr_d
                          ? (double)__builtin_amdgcn_exp2f(fmaf(zd, c, -r.mc_d)) * r.al_d
                          : 0.0;
    return fmax(pt - pd, 0.0);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_resid_part(const uint8_t* __restrict__ tgt,
                                                    const uint8_t* __restrict__ dft, int V,
                                                    int nchunks, float c,
                                                    const SampleRec* __restrict__ rec,
                                                    double* __restrict__ wpart) {
    using Lt = Layout<BF16, VEC>;
    __shared__ double redd[kNT / kWave];
    const int b = blockIdx.x / nchunks;
    const int chunk = blockIdx.x - b * nchunks;
    const SampleRec r = rec[b];
    if (r.mode == MODE_NONE) return;
    const bool resid = r.mode == MODE_RESID;
    float zt[Lt::EPT], zd[Lt::EPT];
    load_chunk<BF16, VEC>(tgt + (size_t)r.row_t * V * Lt::ES, V, chunk * Lt::CH, zt);
    if (resid) {
        load_chunk<BF16, VEC>(dft + (size_t)r.row_d * V * Lt::ES, V, chunk * Lt::CH, zd);
    } else {
#pragma unroll
        for (int i = 0; i < Lt::EPT; ++i) zd[i] = -INFINITY;
    }
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < Lt::EPT; ++i) acc += weight(zt[i], zd[i], r, c, resid);
    acc = block_sum<kNT>(acc, redd);
    if (threadIdx.x == 0) wpart[blockIdx.x] = acc;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kNT) void k_resid_pick(const uint8_t* __restrict__ tgt,
                                                    const uint8_t* __restrict__ dft, int V,
                                                    int nchunks, float c,
                                                    SampleRec* __restrict__ rec,
                                                    const double* __restrict__ wpart,
                                                    int* __restrict__ out_tokens,
                                                    int* __restrict__ err_word,
                                                    double* __restrict__ dbg_mass,
                                                    double* __restrict__ dbg_pick,
                                                    int* __restrict__ dbg_flags) {
    using Lt = Layout<BF16, VEC>;
    __shared__ double redd[kNT / kWave];
    __shared__ int redi[kNT / kWave];
    __shared__ double s_part[1024];
    __shared__ double s_W, s_base, s_wpick;
    __shared__ int s_chunk;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    SampleRec r = rec[b];
    if (r.mode == MODE_NONE) return;
    bool resid = r.mode == MODE_RESID;

    // chunk weights (recomputed here for the fallback, where W = 0 after a rejection)
    for (int q = tid; q < nchunks; q += kNT) s_part[q] = wpart[(size_t)b * nchunks + q];
    __syncthreads();
    if (tid == 0) {
        double W = 0.0;
        for (int q = 0; q < nchunks; ++q) W += s_part[q];
        s_W = W;
    }
    __syncthreads();
    if (resid && !(s_W > 0.0)) {
        // residual mass 0 after a rejection: draw the replacement from p_j instead
        resid = false;
        r.flags |= SPECDEC_ERR_ZFALLBACK;
        for (int q = 0; q < nchunks; ++q) {
            float zt[Lt::EPT];
            load_chunk<BF16, VEC>(tgt + (size_t)r.row_t * V * Lt::ES, V, q * Lt::CH, zt);
            double acc = 0.0;
#pragma unroll
            for (int i = 0; i < Lt::EPT; ++i) acc += weight(zt[i], -INFINITY, r, c, false);
            acc = block_sum<kNT>(acc, redd);
            if (tid == 0) s_part[q] = acc;
        }
        __syncthreads();
        if (tid == 0) {
            double W = 0.0;
            for (int q = 0; q < nchunks; ++q) W += s_part[q];
            s_W = W;
            atomicOr(err_word, SPECDEC_ERR_ZFALLBACK);
        }
        __syncthreads();
    }
    const double W = s_W;
    const double t = (double)r.u * W;
    if (tid == 0) {
        double C = 0.0;
        int q = 0;
        for (; q < nchunks; ++q) {
            if (C + s_part[q] > t) break;
            C += s_part[q];
        }
        if (q == nchunks) {   // unreachable while t < W; keep the last non-empty chunk
            q = nchunks - 1;
            while (q > 0 && !(s_part[q] > 0.0)) --q;
            C = 0.0;
            for (int i = 0; i < q; ++i) C += s_part[i];
        }
        s_chunk = q;
        s_base = C;
    }
    __syncthreads();
    const int chunk = s_chunk;
    const int c0 = chunk * Lt::CH;
    float zt[Lt::EPT], zd[Lt::EPT];
    load_chunk<BF16, VEC>(tgt + (size_t)r.row_t * V * Lt::ES, V, c0, zt);
    if (resid) {
        load_chunk<BF16, VEC>(dft + (size_t)r.row_d * V * Lt::ES, V, c0, zd);
    } else {
#pragma unroll
        for (int i = 0; i < Lt::EPT; ++i) zd[i] = -INFINITY;
    }
    double carry = s_base;
    int found = 0x7fffffff;
    int lastpos = -1;
#pragma unroll
    for (int col = 0; col < Lt::COLS; ++col) {
        double w[Lt::PER], lp[Lt::PER];
        double run = 0.0;
#pragma unroll
        for (int q = 0; q < Lt::PER; ++q) {
            w[q] = weight(zt[col * Lt::PER + q], zd[col * Lt::PER + q], r, c, resid);
            run += w[q];
            lp[q] = run;
        }
        double coltot;
        const double ex = block_excl_scan_d<kNT>(run, redd, &coltot);
        const int i0 = c0 + (col * kNT + tid) * Lt::PER;
        int mine = 0x7fffffff;
#pragma unroll
        for (int q = Lt::PER - 1; q >= 0; --q) {
            if (carry + (ex + lp[q]) > t) mine = i0 + q;
            if (w[q] > 0.0 && i0 + q > lastpos) lastpos = i0 + q;
        }
        found = block_min_i<kNT>(mine, redi);
        if (found != 0x7fffffff) {
            if (i0 <= found && found < i0 + Lt::PER) s_wpick = w[found - i0];
            break;
        }
        carry += coltot;
    }
    if (found == 0x7fffffff) {
        found = block_max_i<kNT>(lastpos, redi);
        if (found >= 0 && tid == 0) {
            s_wpick = weight(load_elem(tgt + (size_t)r.row_t * V * Lt::ES, found, BF16),
                             resid ? load_elem(dft + (size_t)r.row_d * V * Lt::ES, found, BF16)
                                   : -INFINITY,
                             r, c, resid);
        }
    }
    __syncthreads();
    if (tid == 0) {
        out_tokens[r.out_pos] = found;
        if (dbg_mass) dbg_mass[b] = W;
        if (dbg_pick) dbg_pick[b] = s_wpick / W;
        if (dbg_flags) dbg_flags[b] = r.flags;
    }
}

// ---------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsPlan {
    size_t part, rec, wpart, thr, total;
    int nparts, nchunks;
};

static int chunk_elems(int dtype, bool vec) {
    if (dtype == SPECDEC_BF16) return vec ? Layout<true, true>::CH : Layout<true, false>::CH;
    return vec ? Layout<false, true>::CH : Layout<false, false>::CH;
}

static bool topk_active(int top_k, int V) { return top_k > 0 && top_k < V; }

static WsPlan plan_ws(int B, int K, int V, int dtype, int top_k) {
    WsPlan p{};
    // the vector and scalar layouts use the same chunk length
    p.nchunks = (V + chunk_elems(dtype, true) - 1) / chunk_elems(dtype, true);
    p.nparts = topk_active(top_k, V) ? 1 : p.nchunks;
    const size_t rows = (size_t)2 * K + B;
    size_t off = 0;
    p.part = off;
    off = align256(off + rows * p.nparts * sizeof(RowPartial));
    p.rec = off;
    off = align256(off + (size_t)B * sizeof(SampleRec));
    p.wpart = off;
    off = align256(off + (size_t)B * p.nchunks * sizeof(double));
    p.thr = off;
    off = align256(off + rows * sizeof(float));
    p.total = off;
    return p;
}

template <bool BF16, bool VEC>
static void launch_all(const uint8_t* tgt, const uint8_t* dft, int B, int K, int V,
                       int top_k, float c, const WsPlan& p, uint8_t* ws, DecideArgs da,
                       const specdec_debug* dbg, hipStream_t st) {
    const int rows = 2 * K + B;
    RowPartial* part = reinterpret_cast<RowPartial*>(ws + p.part);
    float* thr = reinterpret_cast<float*>(ws + p.thr);
    if (dbg && dbg->ev_stats_begin) hipEventRecord(dbg->ev_stats_begin, st);
    if (topk_active(top_k, V)) {
        hipLaunchKernelGGL((k_topk_rows<BF16, VEC>), dim3(rows), dim3(kTopkNT), 0, st, tgt, dft,
                           K + B, V, top_k, c, part, thr);
    } else if (rows > 0) {
        hipLaunchKernelGGL((k_row_stats<BF16, VEC>), dim3((unsigned)rows * p.nchunks), dim3(kNT),
                           0, st, tgt, dft, K + B, V, p.nchunks, c, part);
    }
    if (dbg && dbg->ev_stats_end) hipEventRecord(dbg->ev_stats_end, st);
    hipLaunchKernelGGL(k_decide, dim3(B), dim3(kWave), 0, st, da);
    SampleRec* rec = reinterpret_cast<SampleRec*>(ws + p.rec);
    double* wpart = reinterpret_cast<double*>(ws + p.wpart);
    hipLaunchKernelGGL((k_resid_part<BF16, VEC>), dim3((unsigned)B * p.nchunks), dim3(kNT), 0, st,
                       tgt, dft, V, p.nchunks, c, rec, wpart);
    hipLaunchKernelGGL((k_resid_pick<BF16, VEC>), dim3(B), dim3(kNT), 0, st, tgt, dft, V,
                       p.nchunks, c, rec, wpart, da.out_tokens, da.err_word,
                       dbg ? dbg->resid_mass : nullptr, dbg ? dbg->picked_prob : nullptr,
                       dbg ? dbg->req_flags : nullptr);
}

}  // namespace sd

extern "C" size_t specdec_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype,
                                                int32_t top_k) {
    if (B < 1 || K < 0 || V < 1 || (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16)) return 0;
    return sd::plan_ws(B, K, V, dtype, top_k).total;
}

extern "C" int specdec_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                              const int32_t* draft_tokens, const int32_t* cu_draft,
                              const float* u_accept, const float* u_sample, int32_t B, int32_t K,
                              int32_t max_k, int32_t V, float temperature, int32_t top_k,
                              int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                              int32_t* err_word, const specdec_debug* dbg, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    using namespace sd;
    if (B < 1 || K < 0 || V < 1 || max_k < 0 || max_k > SPECDEC_MAX_K) return SPECDEC_EINVAL;
    if ((long long)K > (long long)B * max_k) return SPECDEC_EINVAL;
    if (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) return SPECDEC_EINVAL;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return SPECDEC_EINVAL;
    if (!target_logits || !cu_draft || !u_sample || !out_tokens || !num_accepted ||
        !num_emitted || !err_word)
        return SPECDEC_EINVAL;
    if (K > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SPECDEC_EINVAL;
    const WsPlan p = plan_ws(B, K, V, dtype, top_k);
    if ((size_t)(2 * (size_t)K + B) * p.nchunks > 0x7fffffffu || p.nchunks > 1024)
        return SPECDEC_EINVAL;
    if (!workspace || workspace_bytes < p.total || ((uintptr_t)workspace & 15))
        return SPECDEC_EWORKSPACE;

    const double c64 = 1.4426950408889634074 / (double)temperature;   // log2(e) / T
    const float c = (float)c64;
    if (!(c > 0.0f) || !isfinite(c)) return SPECDEC_EINVAL;
    const int es = dtype == SPECDEC_BF16 ? 2 : 4;
    const bool vec = ((size_t)V * es) % 16 == 0 && ((uintptr_t)target_logits & 15) == 0 &&
                     (K == 0 || ((uintptr_t)draft_logits & 15) == 0);
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    const uint8_t* tgt = reinterpret_cast<const uint8_t*>(target_logits);
    const uint8_t* dft = reinterpret_cast<const uint8_t*>(K > 0 ? draft_logits : target_logits);

    DecideArgs da;
    da.tgt = tgt;
    da.dft = dft;
    da.bf16 = dtype == SPECDEC_BF16;
    da.tokens = draft_tokens;
    da.cu = cu_draft;
    da.u_acc = u_accept;
    da.u_smp = u_sample;
    da.B = B;
    da.K = K;
    da.max_k = max_k;
    da.V = V;
    da.nparts = p.nparts;
    da.topk = topk_active(top_k, V);
    da.c = c;
    da.part = reinterpret_cast<const RowPartial*>(ws + p.part);
    da.row_thr = reinterpret_cast<const float*>(ws + p.thr);
    da.out_tokens = out_tokens;
    da.num_acc = num_accepted;
    da.num_emit = num_emitted;
    da.err_word = err_word;
    da.rec = reinterpret_cast<SampleRec*>(ws + p.rec);
    if (dbg) {
        da.dbg = *dbg;
    } else {
        da.dbg = specdec_debug{};
    }
    // the sampling kernel reports flags itself
    da.dbg.req_flags = dbg ? dbg->req_flags : nullptr;

    (void)hipGetLastError();
    if (dtype == SPECDEC_BF16) {
        if (vec) launch_all<true, true>(tgt, dft, B, K, V, top_k, c, p, ws, da, dbg, stream);
        else launch_all<true, false>(tgt, dft, B, K, V, top_k, c, p, ws, da, dbg, stream);
    } else {
        if (vec) launch_all<false, true>(tgt, dft, B, K, V, top_k, c, p, ws, da, dbg, stream);
        else launch_all<false, false>(tgt, dft, B, K, V, top_k, c, p, ws, da, dbg, stream);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_EHIP;
}

extern "C" const char* specdec_status_string(int status) {
    switch (status) {
        case SPECDEC_OK: return "ok";
        case SPECDEC_EINVAL: return "invalid argument";
        case SPECDEC_EHIP: return "HIP runtime error";
        case SPECDEC_EWORKSPACE: return "workspace missing, misaligned or too small";
        default: return "unknown status";
    }
}
