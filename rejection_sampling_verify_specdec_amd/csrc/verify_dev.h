// Device-side bodies of the verification kernels (gfx950), shared by the standalone
// specdec_verify launches and the fused cycle. See verify.hip for the pipeline.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "specdec.h"

namespace sd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNT = 256;        // threads per workgroup of the streaming kernels
constexpr int kVPT = 8;         // 16-byte vectors per thread per chunk

// MODE_PRECISE: a residual draw whose streaming mass came out below kPreciseBelow; the
// pick launch re-derives it with the precise arithmetic (precise_draw)
enum : int { MODE_NONE = 0, MODE_RESID = 1, MODE_BONUS = 2, MODE_PRECISE = 3 };

// Partial statistics of one row chunk (or of a whole row for top-k rows).
struct alignas(16) RowPartial {
    float m;      // max logit of the chunk (-inf if none)
    int nkept;    // kept tokens (top-k rows only)
    double s;     // sum over the chunk of exp2((z - m) * c)
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

// Calls f(z) for this thread's share of a row's V elements, in a fixed order: U 16-byte
// vectors in flight per thread when the row starts 16-byte aligned (the whole vectors),
// single elements otherwise and for the tail. For passes that walk whole rows.
template <bool BF16, int NT, int U, class F>
SD_DEV void walk_row(const uint8_t* __restrict__ row, int V, F&& f) {
    constexpr int EPV = BF16 ? 8 : 4;
    const int tid = threadIdx.x;
    int done = 0;
    if (((uintptr_t)row & 15) == 0) {
        const int nv = V / EPV;
        const u32x4* p = reinterpret_cast<const u32x4*>(row);
        for (int v0 = 0; v0 < nv; v0 += U * NT) {
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * NT + tid;
                x[u] = v < nv ? p[v] : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (v0 + u * NT + tid < nv) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t w = x[u][q];
                        if constexpr (BF16) {
                            f(__uint_as_float(w << 16));
                            f(__uint_as_float(w & 0xffff0000u));
                        } else {
                            f(__uint_as_float(w));
                        }
                    }
                }
            }
        }
        done = nv * EPV;
    }
    for (int i = done + tid; i < V; i += NT) f(load_elem(row, i, BF16));
}

// Element z[col * PER + e] of the calling thread is index c0 + (col * kNT + tid) * PER + e
// of the row; elements at or past V read as -inf.
template <bool BF16, bool VEC>
SD_DEV void load_chunk(const uint8_t* __restrict__ row, int V, int c0,
                       float (&z)[Layout<BF16, VEC>::EPT]) {
    using Lt = Layout<BF16, VEC>;
    const int tid = threadIdx.x;
    if constexpr (VEC) {
        // streamed once: non-temporal loads keep the rows from displacing other lines
        const u32x4* p = reinterpret_cast<const u32x4*>(row);
        u32x4 raw[Lt::COLS];
        const uint32_t fill = BF16 ? 0xff80ff80u : 0xff800000u;
        if (c0 + Lt::CH <= V) {                // whole chunk inside the row
#pragma unroll
            for (int col = 0; col < Lt::COLS; ++col)
                raw[col] = __builtin_nontemporal_load(p + (c0 + (col * kNT + tid) * Lt::PER) / Lt::EPV);
        } else {
#pragma unroll
            for (int col = 0; col < Lt::COLS; ++col) {
                const int i0 = c0 + (col * kNT + tid) * Lt::PER;
                if (i0 < V) {
                    raw[col] = __builtin_nontemporal_load(p + i0 / Lt::EPV);
                } else {
                    raw[col] = (u32x4){fill, fill, fill, fill};
                }
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
// The transform of one row when temperature / top-k / top-p come per request.
constexpr int kRpMode = 3;         // flags & kRpMode: 0 none, 1 top-k (and maybe top-p),
                                   // 2 top-p alone
constexpr int kRpBad = 4;          // the request's parameters are invalid
constexpr int kRpGeneric = 8;      // the row takes the multi-pass select
struct alignas(16) RowParams {
    float c;        // log2(e) / T
    int k;          // the chunk select's k: top_k (mode 1), k_c (mode 2), 0 (mode 0)
    float top_p;
    int flags;
};

template <bool BF16, bool VEC>
SD_DEV void row_stats_body(const uint8_t* __restrict__ tgt, const uint8_t* __restrict__ dft,
                           int rows_t, int V, int nchunks, float c,
                           RowPartial* __restrict__ part, int bid,
                           const RowParams* __restrict__ rpar = nullptr) {
    using Lt = Layout<BF16, VEC>;
    __shared__ float redf[kNT / kWave];
    __shared__ double redd[kNT / kWave];
    __shared__ int redi[kNT / kWave];
    const int row = bid / nchunks;
    const int chunk = bid - row * nchunks;
    if (rpar) c = rpar[row].c;       // per-request temperatures: the row's log2(e) / T
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
        part[bid] = rp;
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

// (hist: 256 u32 of LDS)
template <bool BF16, int NT>
SD_DEV void topk_rows_body(const uint8_t* __restrict__ tgt, const uint8_t* __restrict__ dft,
                           int rows_t, int V, int top_k, float c, RowPartial* __restrict__ part,
                           float* __restrict__ row_thr, int row, unsigned* hist) {
    constexpr int ES = BF16 ? 2 : 4;
    __shared__ float redf[NT / kWave];
    __shared__ double redd[NT / kWave];
    __shared__ int redi[NT / kWave];
    __shared__ uint32_t s_prefix;
    __shared__ int s_krem;
    const uint8_t* base = row_ptr(tgt, dft, rows_t, row, V, ES);
    const int tid = threadIdx.x;

    // pass 0: max, invalid entries (NaN, +inf)
    float mx = -INFINITY;
    int bad = 0;
    walk_row<BF16, NT, 8>(base, V, [&](float z) {
        mx = fmaxf(mx, z);
        bad |= (z != z) | (z == INFINITY);
    });
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
        walk_row<BF16, NT, 8>(base, V, [&](float z) {
            const uint32_t k = f2key(z);
            if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & 0xff], 1u);
        });
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
    int kept = 0;
    walk_row<BF16, NT, 8>(base, V, [&](float z) {
        if (z >= thr && z > -INFINITY) {
            acc += __builtin_amdgcn_exp2f(fmaf(z, c, -mc));
            ++kept;
        }
    });
    const double tot = block_sum<NT>((double)acc, redd);
    kept = block_sum_i<NT>(kept, redi);
    if (tid == 0) {
        RowPartial rp;
        rp.m = m;
        rp.nkept = kept;
        rp.s = bad ? (double)NAN : (m == -INFINITY ? 0.0 : tot * exp2(-(double)emc));
        part[row] = rp;
        row_thr[row] = thr;
    }
}

// ---------------------------------------------------------------------------------------
// Top-k row statistics in two launches, one HBM read per row.
//  chunks: one 256-thread workgroup per 16K-element chunk (8K for fp32), the chunking of the
//    plain statistics kernel. The chunk sits in registers as order-preserving keys (two
//    16-bit keys a register for bf16). Each wave finds the ceil(top_k/4)-th largest of its
//    per-thread max keys (per-16-element-group max keys when top_k > 256) by a ballot radix
//    select, and t_c is the smallest of the four. At least top_k chunk elements are >= t_c,
//    so the row's top_k-th largest element is >= t_c too; the elements >= t_c (for i.i.d. logits a little over top_k per chunk) go
//    to the workspace as (key << 32 | token), one list per wave compacted with ballots
//    (fixed order: register, then lane).
//  merge: one workgroup per row selects the exact top_k-th largest key among the chunks'
//    candidates (their union holds every token the row keeps) and takes max, kept count and
//    exp-sum from the candidates alone. For bf16 target rows it also lists the kept tokens
//    in ascending order (at most kKeptCap): the draw then scans that list instead of the
//    vocabulary.
// Rows holding NaN or +inf, rows with a chunk that overflows its candidate capacity (heavy
// ties at the threshold) and top_k above 1024 take the generic multi-pass select in the
// merge launch instead. -0 and +0 compare equal as floats but not as keys: t_c is lowered
// from key(+0) to key(-0) so that every token the float test keeps is a candidate.
// ---------------------------------------------------------------------------------------
constexpr int kTkNT = kNT;         // threads of a chunk workgroup
constexpr int kTkRegs = kVPT * 4;  // key registers per thread (the chunk's 16-byte vectors)
constexpr int kMergeNT = 128;      // threads of a merge workgroup
constexpr int kTkMaxK = 4 * kTkNT; // largest top_k of the chunked select
constexpr int kTkMaxChunks = 256; // statistics chunks per row at the largest V
constexpr int kTkWaves = kTkNT / kWave;          // candidate lists per chunk
constexpr int kMergeCap = 3072;  // candidates of a row the merge holds in LDS
constexpr int kTkWcapMax = kTkMaxK;   // list capacity at the largest top_k
constexpr int kTkLaneSlots = 7;        // candidates a lane stages before they are listed
constexpr int kTkColumns = (kTkLaneSlots + 1) * kWave;   // a wave's staging (and spill) slots
constexpr int kKeptCap = 512;   // kept tokens of a bf16 target row listed for the draw

struct TopkArgs {
    const uint8_t* tgt;
    const uint8_t* dft;
    int rows_t, V, nchunks, top_k;
    int wcap;                // candidates a wave of a chunk may contribute
    int cstride;             // keys between the lists of consecutive chunks
    int generic;             // 1: every row takes the generic select
    float c;
    int* cnt;                // [rows][nchunks] candidates (-1: NaN / +inf; > 4 * wcap: overflow)
    uint32_t* cand;          // [rows][nchunks] lists of cstride entries: keys (fp32), or
                             // key << 16 | token - chunk start (bf16)
    int* kn;                 // bf16: [rows_t] kept tokens listed (-1: none), else null
    uint32_t* ktok;          // [rows_t][kKeptCap] kept tokens, ascending
    uint16_t* kkey;          // [rows_t][kKeptCap] their keys
    RowPartial* part;        // [rows]
    float* row_thr;          // [rows]
    int topp_mode;           // 0: no top-p; 1: top-p inside the top-k set; 2: top-p alone
    float top_p;
    RowPartial* cpart;       // mode 2: [rows][nchunks] each chunk's max and exp-sum
    uint32_t* ctc;           // mode 2: [rows][nchunks] each chunk's candidate bound t_c
    const struct RowParams* rpar;   // per-request parameters: [rows] each row's, else null
};



// What one chunk workgroup selects, and what one merge workgroup applies.
struct ChunkSel {
    int top_k;      // the chunk's k
    float c;
    bool p2;        // also the chunk's max, exp-sum and bound (top-p alone)
};
struct RowSel {
    int top_k;      // exact top-k select when topp_mode != 2
    int topp_mode;  // 0: no top-p; 1: top-p inside the top-k set; 2: top-p alone
    float top_p;
    float c;
};

// Candidates per row gathered for a top-p row without top-k: the nucleus comes from them
// when the complete upper set they hold carries top_p of the mass, else from full passes.
constexpr int kToppCand = 1024;          // top-p alone: upper-set size per row, about

static inline int topk_wcap(int top_k) { return top_k <= 256 ? 256 : top_k; }
static inline int topk_cstride(int wcap) { return kTkWaves * wcap + 16; }
static_assert(kTkMaxK <= kTkWcapMax, "a list holds top_k keys");
static inline bool topk_generic(int top_k) { return top_k > kTkMaxK; }

template <bool BF16>
struct TopkKeys {
    static constexpr uint32_t KEY_NINF = BF16 ? 0x007fu : 0x007fffffu;     // key(-inf)
    static constexpr uint32_t KEY_PINF = BF16 ? 0xff80u : 0xff800000u;     // key(+inf)
    static constexpr uint32_t KEY_PZERO = BF16 ? 0x8000u : 0x80000000u;    // key(+0)
    static constexpr uint32_t KEY_NZERO = BF16 ? 0x7fffu : 0x7fffffffu;    // key(-0)
    static constexpr uint32_t RAW_NINF = BF16 ? 0xff80ff80u : 0xff800000u;
    static constexpr int KBITS = BF16 ? 16 : 32;
};

typedef short sd_i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short sd_u16x2 __attribute__((ext_vector_type(2)));

// keys of one register: two bf16 (flip all bits of negatives, set the sign of the rest)
// or one fp32
template <bool BF16>
SD_DEV uint32_t reg_keys(uint32_t d) {
    if constexpr (BF16) {
        const sd_i16x2 s = __builtin_bit_cast(sd_i16x2, d) >> (sd_i16x2){15, 15};
        return d ^ (__builtin_bit_cast(uint32_t, s) | 0x80008000u);
    } else {
        return d ^ (uint32_t((int)d >> 31) | 0x80000000u);
    }
}
template <bool BF16>
SD_DEV uint32_t reg_max(uint32_t a, uint32_t b) {
    if constexpr (BF16)
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(sd_u16x2, a),
                                                                      __builtin_bit_cast(sd_u16x2, b)));
    else
        return a > b ? a : b;
}
template <bool BF16>
SD_DEV uint32_t reg_min(uint32_t a, uint32_t b) {
    if constexpr (BF16)
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(sd_u16x2, a),
                                                                      __builtin_bit_cast(sd_u16x2, b)));
    else
        return a < b ? a : b;
}
// the inverse of reg_keys: the raw bits of one register's two bf16 (or one fp32) back from
// their keys (a key with its top bit set is a non-negative value)
template <bool BF16>
SD_DEV uint32_t reg_raw(uint32_t k) {
    if constexpr (BF16) {
        const sd_i16x2 s = __builtin_bit_cast(sd_i16x2, k) >> (sd_i16x2){15, 15};
        return k ^ (~__builtin_bit_cast(uint32_t, s) | 0x80008000u);
    } else {
        return k ^ (~uint32_t((int)k >> 31) | 0x80000000u);
    }
}
template <bool BF16>
SD_DEV float key_to_float(uint32_t k) {
    if constexpr (BF16) {
        const uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
        return __uint_as_float(b << 16);
    } else {
        return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
    }
}

// Called by the 64 threads of wave 0. hist holds 256 bins with at least *krem entries;
// finds the bin d holding the *krem-th largest entry (counting down from bin 255), stores
// d in *dig and *krem minus the entries in bins above d in *krem.
SD_DEV void hist_select(const unsigned* hist, int* dig, int* krem) {
    const int l = threadIdx.x;
    const int k = *krem;
    const unsigned h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
    const int s = int(h0 + h1 + h2 + h3);
    int S = s;                                   // entries in the bins of lanes l..63
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_down(S, o, kWave);
        if (l + o < kWave) S += v;
    }
    int above = S - s;
    if (S >= k && above < k) {
        const unsigned h[4] = {h0, h1, h2, h3};
#pragma unroll
        for (int b = 3; b >= 0; --b) {
            if (above + int(h[b]) >= k) {
                *dig = 4 * l + b;
                *krem = k - above;
                break;
            }
            above += int(h[b]);
        }
    }
}

// P2 (top-p without top-k; 0 never, 1 always, 2 as sel.p2 says): the chunk also writes its
// max and exp-sum (cpart) and its bound t_c (ctc), from which the merge knows the row's
// exp-sum and which candidates are complete.
template <bool BF16, bool VEC, int P2>
SD_DEV void topk_chunk_body(const TopkArgs& a, int row, int chunk, const ChunkSel& sel) {
    const bool p2 = P2 == 2 ? sel.p2 : P2 == 1;
    constexpr int NT = kTkNT;
    constexpr int NR = kTkRegs;
    constexpr int EPR = BF16 ? 2 : 1;                 // elements per register
    using Lt = Layout<BF16, VEC>;
    using Kt = TopkKeys<BF16>;
    static_assert(NR * EPR == Lt::EPT, "a chunk is NT threads x NR registers");
    static_assert(kTkWaves == 4, "t_c takes the minimum of four wave bounds");
    __shared__ uint32_t s_tw[kTkWaves];
    __shared__ float s_mw[kTkWaves];
    __shared__ double s_sw[kTkWaves];
    __shared__ int s_wn[kTkWaves];
    __shared__ uint32_t s_list[kTkWaves * kTkWcapMax];
    const int tid = threadIdx.x;
    const int V = a.V;
    const uint8_t* base = row_ptr(a.tgt, a.dft, a.rows_t, row, V, Lt::ES);
    const int c0 = chunk * Lt::CH;
    // token of element h of register w
    auto token = [&](int w, int h) {
        if constexpr (VEC) return c0 + ((w / 4) * NT + tid) * Lt::EPV + (w % 4) * EPR + h;
        else return c0 + (w * EPR + h) * NT + tid;
    };

    // 1. load (tokens past V read as -inf), keys in place, group max / thread min
    uint32_t r[NR];
    if constexpr (VEC) {
        const u32x4* p = reinterpret_cast<const u32x4*>(base);
#pragma unroll
        for (int j = 0; j < NR / 4; ++j) {
            const int i0 = token(4 * j, 0);
            const u32x4 v = i0 < V ? __builtin_nontemporal_load(p + i0 / Lt::EPV)
                                   : (u32x4){Kt::RAW_NINF, Kt::RAW_NINF, Kt::RAW_NINF, Kt::RAW_NINF};
            r[4 * j] = v.x;
            r[4 * j + 1] = v.y;
            r[4 * j + 2] = v.z;
            r[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int w = 0; w < NR; ++w) {
            if constexpr (BF16) {
                const uint16_t* q = reinterpret_cast<const uint16_t*>(base);
                const int i0 = token(w, 0), i1 = token(w, 1);
                const uint32_t lo = i0 < V ? q[i0] : 0xff80u;
                const uint32_t hi = i1 < V ? q[i1] : 0xff80u;
                r[w] = lo | (hi << 16);
            } else {
                const uint32_t* q = reinterpret_cast<const uint32_t*>(base);
                const int i0 = token(w, 0);
                r[w] = i0 < V ? q[i0] : Kt::RAW_NINF;
            }
        }
    }
    uint32_t gm[4];
    uint32_t kmin = 0xffffffffu;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint32_t m = 0u;
#pragma unroll
        for (int w = g * (NR / 4); w < (g + 1) * (NR / 4); ++w) {
            r[w] = reg_keys<BF16>(r[w]);
            m = reg_max<BF16>(m, r[w]);
            kmin = reg_min<BF16>(kmin, r[w]);
        }
        gm[g] = BF16 ? max(m & 0xffffu, m >> 16) : m;
    }
    if constexpr (BF16) kmin = min(kmin & 0xffffu, kmin >> 16);
    const uint32_t kmax = max(max(gm[0], gm[1]), max(gm[2], gm[3]));
    const int lane = tid % kWave, wv = tid / kWave;
    const bool wbad = __ballot(kmax >= Kt::KEY_PINF || kmin < Kt::KEY_NINF) != 0ull;

    // 2. t_c: every wave takes the ceil(top_k / 4)-th largest of its per-thread (or, when
    //    top_k > 256, per-group) max keys; t_c = the smallest of the four, so each wave, and
    //    the chunk, holds at least top_k elements >= t_c. Upper 16 key bits for fp32.
    const bool groups = sel.top_k > NT;
    const int mth = (sel.top_k + kTkWaves - 1) / kTkWaves;
    uint32_t tv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) tv[g] = BF16 ? gm[g] : gm[g] >> 16;
    const uint32_t tt = BF16 ? kmax : kmax >> 16;
    uint32_t tw = 0u;
    int krem = mth;
#pragma unroll
    for (int b = 15; b >= 0; --b) {
        const uint32_t probe = (tw | (1u << b)) >> b;
        int n;
        if (groups) {
            n = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) n += __popcll(__ballot((tv[g] >> b) == probe));
        } else {
            n = __popcll(__ballot((tt >> b) == probe));
        }
        if (n >= krem) tw |= 1u << b;
        else krem -= n;
    }
    if (lane == 0) s_tw[wv] = tw;
    if (P2 != 0 && p2) {
        // top-p without top-k also needs the row's exp-sum: each wave sums exp2((z - m_w) c)
        // over its elements with its own max m_w; thread 0 combines the four in fp64
        const uint32_t wk = uint32_t(wave_max_i(int(kmax ^ 0x80000000u))) ^ 0x80000000u;
        const float mw = key_to_float<BF16>(BF16 ? (wk & 0xffffu) : wk);
        double sw = 0.0;
        if (mw > -INFINITY && !wbad) {
            const float mc = mw * sel.c;
            const float emc = fmaf(mw, sel.c, -mc);
            // fp32 trees of 16 (8) terms per register group, then across the groups
            float gs[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float e[NR / 4 * EPR];
#pragma unroll
                for (int w = 0; w < NR / 4; ++w) {
                    // the values back from the keys, both halves of a register at once
                    const uint32_t raw = reg_raw<BF16>(r[g * (NR / 4) + w]);
#pragma unroll
                    for (int h = 0; h < EPR; ++h) {
                        const float z = __uint_as_float(
                            BF16 ? (h ? raw & 0xffff0000u : raw << 16) : raw);
                        e[w * EPR + h] = __builtin_amdgcn_exp2f(fmaf(z, sel.c, -mc));
                    }
                }
                gs[g] = tree_sum(e);
            }
            sw = wave_sum((double)tree_sum(gs)) * exp2(-(double)emc);
        }
        if (lane == 0) {
            s_mw[wv] = mw;
            s_sw[wv] = sw;
        }
    }
    __syncthreads();
    uint32_t t0 = min(min(s_tw[0], s_tw[1]), min(s_tw[2], s_tw[3]));
    if constexpr (!BF16) t0 <<= 16;
    if (t0 == Kt::KEY_PZERO) t0 = Kt::KEY_NZERO;
    if (P2 != 0 && p2 && tid == 0) {
        float mcx = s_mw[0];
        for (int i = 1; i < kTkWaves; ++i) mcx = fmaxf(mcx, s_mw[i]);
        double sc = 0.0;
        if (mcx > -INFINITY)
            for (int i = 0; i < kTkWaves; ++i)
                if (s_mw[i] > -INFINITY)
                    sc += s_sw[i] * exp2(((double)s_mw[i] - (double)mcx) * (double)sel.c);
        RowPartial rp;
        rp.m = mcx;
        rp.nkept = 0;
        rp.s = sc;
        const size_t ci = (size_t)row * a.nchunks + chunk;
        a.cpart[ci] = rp;
        a.ctc[ci] = t0;
    }

    // 3. candidates (key >= t0): each wave fills its own list, then copies it out with
    //    coalesced stores. Candidates are few, so each lane first stages its own in a column
    //    of kTkLaneSlots LDS slots (slot-major: a wave's column writes hit distinct banks)
    //    and a wave scan of the lane counts places them; a wave with a fuller lane, or lists
    //    too long to leave room for the columns, compacts with one ballot per element
    uint32_t* lst = s_list + wv * a.wcap;
    auto entry = [&](uint32_t k, int w, int h) {
        return BF16 ? (k << 16) | (uint32_t)(token(w, h) - c0) : k;
    };
    int woff = 0;
    bool staged = kTkWaves * (a.wcap + kTkColumns) <= kTkWaves * kTkWcapMax;
    if (staged) {
        uint32_t* col = s_list + kTkWaves * a.wcap + wv * kTkColumns + lane;
        int ns = 0;                                      // this lane's staged candidates
#pragma unroll
        for (int w = 0; w < NR; ++w)
#pragma unroll
            for (int h = 0; h < EPR; ++h) {
                const uint32_t k = (r[w] >> (16 * h)) & (BF16 ? 0xffffu : ~0u);
                if (k >= t0) {
                    col[min(ns, kTkLaneSlots) * kWave] = entry(k, w, h);   // slot 7: spill
                    ++ns;
                }
            }
        staged = __ballot(ns > kTkLaneSlots) == 0ull;
        if (staged) {
            int p = ns;                                  // exclusive scan of the lane counts
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int y = __shfl_up(p, o, kWave);
                if (lane >= o) p += y;
            }
            woff = __shfl(p, kWave - 1, kWave);
            p -= ns;
#pragma unroll
            for (int j = 0; j < kTkLaneSlots; ++j)
                if (j < ns && p + j < a.wcap) lst[p + j] = col[j * kWave];
        }
    }
    if (!staged) {
        woff = 0;
#pragma unroll
        for (int w = 0; w < NR; ++w)
#pragma unroll
            for (int h = 0; h < EPR; ++h) {
                const uint32_t k = (r[w] >> (16 * h)) & (BF16 ? 0xffffu : ~0u);
                const bool f = k >= t0;
                const uint64_t bal = __ballot(f);
                if (bal) {
                    const int pos = woff + (int)__builtin_amdgcn_mbcnt_hi(
                                               uint32_t(bal >> 32),
                                               __builtin_amdgcn_mbcnt_lo(uint32_t(bal), 0u));
                    if (f && pos < a.wcap) lst[pos] = entry(k, w, h);
                    woff += __popcll(bal);
                }
            }
    }
    if (lane == 0) s_wn[wv] = wbad ? -1 : woff;
    __syncthreads();
    int before = 0, total = 0, bad = 0, over = 0;
#pragma unroll
    for (int i = 0; i < kTkWaves; ++i) {
        const int n = s_wn[i];
        before += i < wv ? n : 0;
        total += n;
        bad |= n < 0;
        over |= n > a.wcap;
    }
    const size_t ci = (size_t)row * a.nchunks + chunk;
    if (!bad && !over) {
        uint32_t* out = a.cand + ci * a.cstride + before;
        for (int i = lane; i < woff; i += kWave) out[i] = lst[i];
    }
    if (tid == 0) a.cnt[ci] = bad ? -1 : (over ? kTkWaves * a.wcap + 1 : total);
}

// Top-p mass in fixed point: exp2(z c - m c) in units of 2^-42, rounded, so that sums do
// not depend on the order of the adds (a row of 2^21 weights <= 1 stays below 2^63).
constexpr double kMassFix = 4398046511104.0;

SD_DEV unsigned long long mass_fix(float w) { return (unsigned long long)((double)w * kMassFix + 0.5); }

// Called by the 64 threads of wave 0. hist holds NB bins of fixed-point mass (NB / 64 per
// lane). The mass to reach is frac * (all of hist) when frac > 0, else *need. Finds the
// largest bin d whose suffix mass (bins d..NB-1) reaches it; leaves d in *dig and the mass
// still to reach inside bin d in *need; *dig = -1 when the whole histogram is short of it.
template <int NB>
SD_DEV void hist_select_mass(const unsigned long long* hist, int* dig, double* need, double frac) {
    constexpr int BPL = NB / kWave;
    static_assert(BPL * kWave == NB, "whole bins per lane");
    const int l = threadIdx.x;
    unsigned long long own = 0ull;
#pragma unroll
    for (int b = 0; b < BPL; ++b) own += hist[BPL * l + b];
    unsigned long long S = own;                  // mass of the bins of lanes l..63
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const unsigned long long v = __shfl_down(S, o, kWave);
        if (l + o < kWave) S += v;
    }
    const double nd = frac > 0.0 ? frac * (double)__shfl(S, 0, kWave) : *need;
    unsigned long long above = S - own;
    if (l == 0 && (double)S < nd) *dig = -1;
    if ((double)S >= nd && (double)above < nd) {
        for (int b = BPL - 1; b >= 0; --b) {
            const unsigned long long h = hist[BPL * l + b];
            if ((double)(above + h) >= nd) {
                *dig = BPL * l + b;
                *need = nd - (double)above;
                break;
            }
            above += h;
        }
    }
}

// Nucleus boundary key over a set of keys: the largest key K such that the keys >= K carry
// frac of the mass of the keys >= lo (frac > 0), or need0 of it in fixed point (frac = 0).
// One digit of up to DBITS bits per pass over the set, most significant first, from a
// histogram of NB >= 2^DBITS bins; each(f) calls f(key, z) for this thread's share of the
// set (canonical keys: -0 as +0). Returns false (K undefined) when the mass of the keys
// >= lo is short of need0. All NT threads call it; h64: NB u64 of LDS.
template <int NT, int KBITS, int DBITS, int NB, class Each>
SD_DEV bool nucleus_key(Each each, uint32_t lo, float c, float mc, double frac, double need0,
                        unsigned long long* h64, uint32_t* K) {
    static_assert((1 << DBITS) <= NB, "a digit's bins fit the histogram");
    __shared__ int s_dig;
    __shared__ double s_need;
    const int tid = threadIdx.x;
    if (tid == 0) s_need = need0;
    uint32_t prefix = 0u;
    for (int hi = KBITS; hi > 0; hi -= DBITS) {
        const int lb = hi > DBITS ? hi - DBITS : 0;
        const uint32_t hmask = hi >= KBITS ? 0u : ~0u << hi;
        const uint32_t dmask = (1u << (hi - lb)) - 1u;
        for (int i = tid; i < NB; i += NT) h64[i] = 0ull;
        __syncthreads();
        each([&](uint32_t k, float z) {
            if (k >= lo && (k & hmask) == prefix)
                atomicAdd(&h64[(k >> lb) & dmask],
                          mass_fix(__builtin_amdgcn_exp2f(fmaf(z, c, -mc))));
        });
        __syncthreads();
        if (tid < kWave) hist_select_mass<NB>(h64, &s_dig, &s_need, hi == KBITS ? frac : 0.0);
        __syncthreads();
        const int d = s_dig;
        if (d < 0) return false;
        prefix |= (uint32_t)d << lb;
    }
    *K = prefix;
    return true;
}

// Nucleus of one row by full passes over it (rows that took the generic top-k select, or
// whose nucleus reaches below the gathered candidates): the boundary over the tokens with
// logit >= thr_lo (finite), then the kept count and exp-sum in a last pass. m: the row max.
// The first digit has 10 bits (sign, exponent, one mantissa bit for bf16) so that the
// histogram adds of a wave spread over many bins. h64: kToppRowBins u64 of LDS.
constexpr int kToppRowDigit = 10;
constexpr int kToppRowBins = 1024;
template <bool BF16, int NT>
SD_DEV void topp_rows_body(const TopkArgs& a, int row, float m, float thr_lo, float c,
                           float top_p, unsigned long long* h64) {
    using Kt = TopkKeys<BF16>;
    constexpr int ES = BF16 ? 2 : 4;
    __shared__ double redd[NT / kWave];
    __shared__ int redi[NT / kWave];
    const int tid = threadIdx.x;
    const uint8_t* base = row_ptr(a.tgt, a.dft, a.rows_t, row, a.V, ES);
    const float mc = m * c;
    const float emc = fmaf(m, c, -mc);
    auto keyz = [](float z) {                    // canonical key of a logit (-0 as +0)
        const uint32_t k = BF16 ? f2key(z) >> 16 : f2key(z);
        return k == Kt::KEY_NZERO ? Kt::KEY_PZERO : k;
    };
    const uint32_t lo = max(thr_lo > -INFINITY ? keyz(thr_lo) : 0u, Kt::KEY_NINF + 1u);
    uint32_t K = lo;
    const bool ok = nucleus_key<NT, Kt::KBITS, kToppRowDigit, kToppRowBins>(
        [&](auto f) {
            walk_row<BF16, NT, 8>(base, a.V, [&](float z) {
                if (z > -INFINITY) f(keyz(z), z);
            });
        },
        lo, c, mc, (double)top_p, 0.0, h64, &K);
    const float thr = key_to_float<BF16>(ok ? max(K, lo) : lo);
    float acc = 0.f;
    int kept = 0;
    walk_row<BF16, NT, 8>(base, a.V, [&](float z) {
        if (z >= thr && z > -INFINITY) {
            acc += __builtin_amdgcn_exp2f(fmaf(z, c, -mc));
            ++kept;
        }
    });
    const double tot = block_sum<NT>((double)acc, redd);
    kept = block_sum_i<NT>(kept, redi);
    if (tid == 0) {
        RowPartial rp;
        rp.m = m;
        rp.nkept = kept;
        rp.s = tot * exp2(-(double)emc);
        a.part[row] = rp;
        a.row_thr[row] = thr;
    }
}

// Bins 0 .. NB-1 of token counts in descending key order, bin i weighing wt(i, count) (an
// exact integer: the count itself, or the count times the fixed-point mass of the bin's
// key): the first bin at which the running weight reaches need (frac > 0: frac times the
// total weight). Returns NB when the total falls short. All NT threads call; red holds
// NT / 64 u64 of LDS; the caller synchronizes before it writes cnt again.
template <int NT, int NB, class Wt>
SD_DEV int first_bin_reaching(const unsigned* cnt, Wt wt, double frac, double need,
                              unsigned long long* red, int* s_bin) {
    constexpr int BPT = NB / NT;
    static_assert(BPT * NT == NB, "whole bins per thread");
    const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
    unsigned long long own = 0ull, bm[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        const unsigned n = cnt[tid * BPT + j];
        bm[j] = n ? wt(tid * BPT + j, n) : 0ull;
        own += bm[j];
    }
    unsigned long long x = own;                          // inclusive scan over the threads
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const unsigned long long y = __shfl_up(x, o, kWave);
        if (l >= o) x += y;
    }
    if (l == kWave - 1) red[w] = x;
    if (tid == 0) *s_bin = NB;
    __syncthreads();
    unsigned long long before = x - own, total = 0ull;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        before += i < w ? red[i] : 0ull;
        total += red[i];
    }
    const double nd = frac > 0.0 ? frac * (double)total : need;
    if ((double)(before + own) >= nd && (double)before < nd) {
        unsigned long long acc = before;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            acc += bm[j];
            if ((double)acc >= nd) {
                *s_bin = tid * BPT + j;
                break;
            }
        }
    }
    __syncthreads();
    return *s_bin;
}

// Top-p alone, bf16, when the candidates' complete upper set (keys >= lo) is short of the
// nucleus: every bf16 key is one logit value, so one pass that counts the row's tokens on
// each of the 1024 keys below lo finds the boundary exactly, each key's mass being its
// count times one exponential (the same fixed-point mass the per-token sums use), and the
// kept sum follows from the counts without another pass. keys[0 .. total) are the row's
// candidate entries (key << 16 | offset); need is the nucleus mass in fixed point, in
// units of exp2(z c - mc); s_cnt: kToppBelow u32 of LDS (bin i: key lo - 1 - i). Returns
// false, having written nothing, when the boundary lies further below (the caller then runs
// the full-row passes).
constexpr int kToppBelow = 1024;
template <int NT>
SD_DEV bool topp_below_bf16(const TopkArgs& a, int row, float m, float mc, float emc, float c,
                            uint32_t lo, double need, const uint32_t* keys, int total,
                            unsigned* s_cnt) {
    using Kt = TopkKeys<true>;
    constexpr int BPT = kToppBelow / NT;
    static_assert(BPT * NT == kToppBelow, "whole bins per thread");
    __shared__ unsigned long long s_red[NT / kWave];
    __shared__ double redd[NT / kWave];
    __shared__ int redi[NT / kWave];
    __shared__ int s_bin;
    const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
    auto canon = [](uint32_t k) { return k == Kt::KEY_NZERO ? Kt::KEY_PZERO : k; };
    auto zof = [](uint32_t k) { return key_to_float<true>(k); };
    // 1. the upper set's mass, in the nucleus' fixed point
    unsigned long long up = 0ull;
    for (int i = tid; i < total; i += NT) {
        const uint32_t k = canon(keys[i] >> 16);
        if (k >= lo) up += mass_fix(__builtin_amdgcn_exp2f(fmaf(zof(k), c, -mc)));
    }
    up = wave_sum_u64(up);
    if (l == 0) s_red[w] = up;
    for (int i = tid; i < kToppBelow; i += NT) s_cnt[i] = 0u;
    __syncthreads();
    up = 0ull;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) up += s_red[i];
    const double need2 = need - (double)up;
    // 2. one pass: tokens per key in [lo - 1024, lo)
    const uint32_t kfloor = lo > Kt::KEY_NINF + 1u + kToppBelow ? lo - kToppBelow : Kt::KEY_NINF + 1u;
    const uint8_t* base = row_ptr(a.tgt, a.dft, a.rows_t, row, a.V, 2);
    walk_row<true, NT, 8>(base, a.V, [&](float z) {
        const uint32_t k = canon(f2key(z) >> 16);
        if (k < lo && k >= kfloor) atomicAdd(&s_cnt[lo - 1u - k], 1u);
    });
    __syncthreads();
    // 3. the first bin (descending keys) whose cumulative mass reaches need2
    unsigned long long own = 0ull, bm[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        const int i = tid * BPT + j;
        const uint32_t k = lo - 1u - (uint32_t)i;
        bm[j] = (k >= kfloor && s_cnt[i]) ?
                    (unsigned long long)s_cnt[i] * mass_fix(__builtin_amdgcn_exp2f(fmaf(zof(k), c, -mc))) : 0ull;
        own += bm[j];
    }
    unsigned long long x = own;                          // inclusive scan over threads
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const unsigned long long y = __shfl_up(x, o, kWave);
        if (l >= o) x += y;
    }
    if (l == kWave - 1) s_red[w] = x;
    if (tid == 0) s_bin = kToppBelow;
    __syncthreads();
    unsigned long long before = x - own;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) before += i < w ? s_red[i] : 0ull;
    if ((double)(before + own) >= need2 && (double)before < need2) {
        unsigned long long acc = before;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            acc += bm[j];
            if ((double)acc >= need2) {
                s_bin = tid * BPT + j;
                break;
            }
        }
    }
    __syncthreads();
    const int bin = s_bin;
    if (bin >= kToppBelow || lo - 1u - (uint32_t)bin < kfloor) return false;
    const uint32_t K = lo - 1u - (uint32_t)bin;
    // 4. kept count and exp-sum: the upper set's candidates, then the bins down to K
    float accf = 0.f;
    int kept = 0;
    for (int i = tid; i < total; i += NT) {
        const uint32_t k = canon(keys[i] >> 16);
        if (k >= lo) {
            accf += __builtin_amdgcn_exp2f(fmaf(zof(k), c, -mc));
            ++kept;
        }
    }
    double accd = (double)accf;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        const int i = tid * BPT + j;
        if (i <= bin && s_cnt[i]) {
            const uint32_t k = lo - 1u - (uint32_t)i;
            accd += (double)s_cnt[i] * (double)__builtin_amdgcn_exp2f(fmaf(zof(k), c, -mc));
            kept += (int)s_cnt[i];
        }
    }
    const double tot = block_sum<NT>(accd, redd);
    kept = block_sum_i<NT>(kept, redi);
    if (tid == 0) {
        RowPartial rp;
        rp.m = m;
        rp.nkept = kept;
        rp.s = tot * exp2(-(double)emc);
        a.part[row] = rp;
        a.row_thr[row] = zof(K);
    }
    return true;
}

template <bool BF16, int NT>
SD_DEV void topk_merge_body(const TopkArgs& a, int row, const RowSel& sel) {
    constexpr int LPT = kTkMaxChunks > NT ? kTkMaxChunks / NT : 1;   // lists per thread
    constexpr int UNR = 8;                              // candidate loads in flight per thread
    using Kt = TopkKeys<BF16>;
    // 4 KB of LDS for one use at a time: per-key token counts, the digit histograms, the
    // count bins below the candidates, then the kept tokens and their keys
    constexpr int kRangeBins = 1024;
    __shared__ __attribute__((aligned(16))) uint32_t s_work[kRangeBins];
    static_assert(kKeptCap * 6 <= kRangeBins * 4 && kToppBelow <= kRangeBins &&
                      256 * 8 <= kRangeBins * 4, "the uses of the work area fit");
    unsigned* hist = s_work;
    uint32_t* s_ktok = s_work;
    uint16_t* s_kkey = reinterpret_cast<uint16_t*>(s_work + kKeptCap);
    __shared__ int s_off[kTkMaxChunks + 1];
    __shared__ __attribute__((aligned(16))) uint32_t keys[kMergeCap];   // entries as the chunks
                                                                     // wrote them
    static_assert(kMergeCap * 4 >= kToppRowBins * 8, "the full-row nucleus histogram fits");
    static_assert(kMergeCap >= 2 * kTkMaxChunks, "the chunks' run bounds fit over the candidates");
    __shared__ int redi[NT / kWave];
    __shared__ double redd[2 * (NT / kWave)];
    __shared__ unsigned long long s_red64[NT / kWave];
    __shared__ int s_dig, s_krem, s_bin;
    __shared__ unsigned s_kmax, s_kmin;
    // an entry's key
    auto key_of = [](uint32_t e) { return BF16 ? e >> 16 : e; };
    const bool listed = BF16 && a.kn && row < a.rows_t;
    const int tid = threadIdx.x;
    const int nl = a.nchunks;
    const int lcap = kTkWaves * a.wcap;
    // list counts (thread t owns lists t*LPT ..); a bad or overflowing list pushes the
    // total past the LDS capacity, which sends the row to the generic select
    int cnt[LPT];
    int mine = 0;
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
        const int l = tid * LPT + q;
        cnt[q] = (!a.generic && l < nl) ? a.cnt[(size_t)row * nl + l] : 0;
        mine += (cnt[q] < 0 || cnt[q] > lcap) ? kMergeCap + 1 : cnt[q];
    }
    if (a.generic) mine = kMergeCap + 1;
    if (tid == 0) {
        s_krem = sel.top_k;
        s_kmax = 0u;
        s_kmin = ~0u;
    }
    int total;
    int off = block_excl_scan_i<NT>(mine, redi, &total);
    if (total > kMergeCap) {
        if (listed && tid == 0) a.kn[row] = -1;
        // generic select (all of the row's finite tokens for top-p alone), then the nucleus
        topk_rows_body<BF16, NT>(a.tgt, a.dft, a.rows_t, a.V, sel.topp_mode == 2 ? a.V : sel.top_k,
                                 sel.c, a.part, a.row_thr, row, s_work);
        if (sel.topp_mode) {
            // the row max and validity as the select left them (tid 0 wrote them)
            if (tid == 0) {
                const RowPartial rp = a.part[row];
                s_kmax = (rp.s == rp.s && rp.m > -INFINITY) ? 1u : 0u;
                redd[0] = rp.m;
                redd[1] = a.row_thr[row];
            }
            __syncthreads();
            const bool run = s_kmax != 0u;
            const float rm = (float)redd[0], tk = (float)redd[1];
            __syncthreads();
            if (run)
                topp_rows_body<BF16, NT>(a, row, rm, sel.topp_mode == 1 ? tk : -INFINITY, sel.c,
                                         sel.top_p, reinterpret_cast<unsigned long long*>(keys));
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
        const int l = tid * LPT + q;
        if (l < nl) s_off[l] = off;
        off += cnt[q];
    }
    if (tid == 0) s_off[nl] = total;
    __syncthreads();

    // candidate keys into LDS: entry e of the row lives in the list l with
    // s_off[l] <= e < s_off[l + 1]
    const uint32_t* cand = a.cand + (size_t)row * nl * a.cstride;
    auto list_of = [&](int e) {        // largest l with s_off[l] <= e
        int lo = 0, hi = nl;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= e) lo = mid;
            else hi = mid;
        }
        return lo;
    };
    uint32_t kmax = 0u, kmin = ~0u;
    for (int e0 = 0; e0 < total; e0 += UNR * NT) {
        uint32_t v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int e = e0 + u * NT + tid;
            v[u] = 0u;
            if (e < total) {
                const int lo = list_of(e);
                v[u] = cand[(size_t)lo * a.cstride + (e - s_off[lo])];
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int e = e0 + u * NT + tid;
            if (e < total) {
                keys[e] = v[u];
                kmax = max(kmax, key_of(v[u]));
                kmin = min(kmin, key_of(v[u]));
            }
        }
    }
    // the candidates' key range (wave reductions, then one LDS atomic per wave)
    kmax = uint32_t(wave_max_i(int(kmax ^ 0x80000000u))) ^ 0x80000000u;
    kmin = uint32_t(wave_min_i(int(kmin ^ 0x80000000u))) ^ 0x80000000u;
    if (tid % kWave == 0) {
        if (kmax) atomicMax(&s_kmax, kmax);
        atomicMin(&s_kmin, kmin);
    }
    __syncthreads();
    const uint32_t khi = s_kmax, klo = s_kmin;

    // exact top_k-th largest candidate key (no top-k: none). Candidates cluster on a few
    // high digits, so histograms of digits funnel their adds into a few bins; when the
    // candidates' keys span fewer than kRangeBins values (the rule for bf16 rows) one pass
    // counts the tokens on each key and the key follows from the counts; else one 8-bit
    // digit at a time
    uint32_t prefix = 0u;
    if (sel.topp_mode != 2 && khi >= klo && khi - klo < (uint32_t)kRangeBins) {
        for (int i = tid; i < kRangeBins; i += NT) hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < total; i += NT) atomicAdd(&hist[khi - key_of(keys[i])], 1u);
        __syncthreads();
        const int bin = first_bin_reaching<NT, kRangeBins>(
            hist, [](int, unsigned n) { return (unsigned long long)n; }, 0.0, (double)sel.top_k,
            s_red64, &s_bin);
        prefix = bin < kRangeBins ? khi - (uint32_t)bin : Kt::KEY_NINF;
        __syncthreads();
    } else if (sel.topp_mode != 2) {
#pragma unroll
        for (int shift = Kt::KBITS - 8; shift >= 0; shift -= 8) {
            const uint32_t hmask = shift + 8 >= Kt::KBITS ? 0u : ~0u << (shift + 8);
            for (int i = tid; i < 256; i += NT) hist[i] = 0u;
            __syncthreads();
            for (int i = tid; i < total; i += NT) {
                const uint32_t k = key_of(keys[i]);
                if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & 0xffu], 1u);
            }
            __syncthreads();
            if (tid < kWave) hist_select(hist, &s_dig, &s_krem);
            __syncthreads();
            prefix |= (uint32_t)s_dig << shift;
        }
    }
    float thr = sel.topp_mode == 2 ? -INFINITY : key_to_float<BF16>(prefix);
    const float m = key_to_float<BF16>(khi);
    const float mc = m * sel.c;
    const float emc = fmaf(m, sel.c, -mc);
    if (sel.topp_mode && m > -INFINITY) {
        // top-p: the nucleus boundary among the candidates (-0 ranks with +0, as the float
        // comparisons do)
        auto canon = [](uint32_t k) { return k == Kt::KEY_NZERO ? Kt::KEY_PZERO : k; };
        uint32_t lo;
        double frac = 0.0, need = 0.0;
        if (sel.topp_mode == 1) {
            // with top-k: the kept set is every candidate >= the top-k threshold
            lo = max(canon(prefix), Kt::KEY_NINF + 1u);
            frac = (double)sel.top_p;
        } else {
            // no top-k: the row's exp-sum from the chunk partials; the candidates hold the
            // complete upper set above every chunk's bound t_c
            double sp = 0.0;
            uint32_t tg = 0u;
#pragma unroll
            for (int q = 0; q < LPT; ++q) {
                const int l = tid * LPT + q;
                if (l < nl) {
                    const RowPartial cp = a.cpart[(size_t)row * nl + l];
                    if (cp.m > -INFINITY)
                        sp += cp.s * exp2(((double)cp.m - (double)m) * (double)sel.c);
                    tg = max(tg, a.ctc[(size_t)row * nl + l]);
                }
            }
            const double S = block_sum<NT>(sp, redd);
            tg = uint32_t(block_max_i<NT>(int(tg ^ 0x80000000u), redi)) ^ 0x80000000u;
            lo = (tg == Kt::KEY_PZERO || tg == Kt::KEY_NZERO) ? Kt::KEY_PZERO + 1u : canon(tg);
            lo = max(lo, Kt::KEY_NINF + 1u);
            need = (double)sel.top_p * S * exp2((double)emc) * kMassFix;
        }
        uint32_t K = lo;
        bool ok = false;
        const uint32_t chi = canon(khi);
        if (chi >= lo && chi - lo < (uint32_t)kRangeBins) {
            // every key is one value: the tokens on each key >= lo, then each bin's mass as
            // its count times one exponential (the fixed-point mass of its key)
            for (int i = tid; i < kRangeBins; i += NT) hist[i] = 0u;
            __syncthreads();
            for (int i = tid; i < total; i += NT) {
                const uint32_t k = canon(key_of(keys[i]));
                if (k >= lo) atomicAdd(&hist[chi - k], 1u);
            }
            __syncthreads();
            const int bin = first_bin_reaching<NT, kRangeBins>(
                hist,
                [&](int i, unsigned n) {
                    const float z = key_to_float<BF16>(chi - (uint32_t)i);
                    return (unsigned long long)n *
                           mass_fix(__builtin_amdgcn_exp2f(fmaf(z, sel.c, -mc)));
                },
                frac, need, s_red64, &s_bin);
            ok = bin < kRangeBins;
            K = chi - (uint32_t)bin;
        } else if (chi >= lo) {
            ok = nucleus_key<NT, Kt::KBITS, 8, 256>(
                [&](auto f) {
                    for (int i = tid; i < total; i += NT) {
                        const uint32_t k = canon(key_of(keys[i]));
                        f(k, key_to_float<BF16>(k));
                    }
                },
                lo, sel.c, mc, frac, need, reinterpret_cast<unsigned long long*>(s_work), &K);
        }
        if (!ok && sel.topp_mode == 2) {
            // the nucleus reaches below the candidates: for bf16 first one counting pass
            // over the keys just below them, else (or when it reaches further) full passes
            if (listed && tid == 0) a.kn[row] = -1;
            __syncthreads();
            if constexpr (BF16) {
                if (topp_below_bf16<NT>(a, row, m, mc, emc, sel.c, lo, need, keys, total, s_work))
                    return;
            }
            topp_rows_body<BF16, NT>(a, row, m, -INFINITY, sel.c, sel.top_p,
                                     reinterpret_cast<unsigned long long*>(keys));
            return;
        }
        thr = key_to_float<BF16>(ok ? max(K, lo) : lo);
        __syncthreads();                    // the histogram memory holds kept tokens next
    }
    // kept count and exp-sum; thread t takes the candidates [t q, t q + q), so that a
    // workgroup scan of the kept counts lists the kept tokens in candidate order
    const int q = (total + NT - 1) / NT;
    const int i0 = min(tid * q, total), i1 = min(i0 + q, total);
    auto is_kept = [&](float z) { return z >= thr && z > -INFINITY; };
    constexpr int KU = 4;                   // candidate reads in flight per thread
    float acc = 0.f;
    int kept = 0;
    for (int i = i0; i < i1; i += KU) {
        uint32_t e[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) e[u] = i + u < i1 ? keys[i + u] : 0u;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const float z = key_to_float<BF16>(key_of(e[u]));
            if (i + u < i1 && is_kept(z)) {
                acc += __builtin_amdgcn_exp2f(fmaf(z, sel.c, -mc));
                ++kept;
            }
        }
    }
    if (listed) {
        // the kept tokens in ascending order. Candidate order is chunk order, so the kept
        // tokens of one chunk form one run and the runs ascend: a token's rank is the start
        // of its chunk's run plus its rank within the run
        constexpr uint32_t CH = Layout<BF16, true>::CH;
        int nk;
        int pos = block_excl_scan_i<NT>(kept, redi, &nk);
        if (nk <= kKeptCap) {
            for (int i = i0; i < i1; i += KU) {
                uint32_t e[KU];
#pragma unroll
                for (int u = 0; u < KU; ++u) e[u] = i + u < i1 ? keys[i + u] : 0u;
#pragma unroll
                for (int u = 0; u < KU; ++u) {
                    const uint32_t k = key_of(e[u]);
                    if (i + u < i1 && is_kept(key_to_float<BF16>(k))) {
                        s_ktok[pos] = (uint32_t)list_of(i + u) * CH + (e[u] & 0xffffu);
                        s_kkey[pos] = (uint16_t)k;
                        ++pos;
                    }
                }
            }
        }
        __syncthreads();                    // the candidates are no longer read
        if (nk <= kKeptCap) {
            int* run_lo = reinterpret_cast<int*>(keys);         // per chunk: its run's bounds
            int* run_hi = run_lo + kTkMaxChunks;
            for (int p = tid; p < nk; p += NT) {
                const uint32_t c = s_ktok[p] / CH;
                if (p == 0 || s_ktok[p - 1] / CH != c) run_lo[c] = p;
                if (p == nk - 1 || s_ktok[p + 1] / CH != c) run_hi[c] = p + 1;
            }
            __syncthreads();
            for (int p = tid; p < nk; p += NT) {
                const uint32_t x = s_ktok[p];
                const int lo = run_lo[x / CH], hi = run_hi[x / CH];
                int rank = lo, j = lo;
                for (; j < hi && (j & 3); ++j) rank += s_ktok[j] < x;
                for (; j + 16 <= hi; j += 16) {         // four 16-byte reads in flight
                    uint32_t t[16];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const uint4 v = *reinterpret_cast<const uint4*>(s_ktok + j + 4 * g);
                        t[4 * g] = v.x;
                        t[4 * g + 1] = v.y;
                        t[4 * g + 2] = v.z;
                        t[4 * g + 3] = v.w;
                    }
#pragma unroll
                    for (int g = 0; g < 16; ++g) rank += t[g] < x;
                }
                for (; j < hi; ++j) rank += s_ktok[j] < x;
                a.ktok[(size_t)row * kKeptCap + rank] = x;
                a.kkey[(size_t)row * kKeptCap + rank] = s_kkey[p];
            }
        }
        if (tid == 0) a.kn[row] = nk <= kKeptCap ? nk : -1;
    }
    // kept count and sum in one reduction (a count below 2^53 is exact in fp64)
    double sum = wave_sum((double)acc), kd = wave_sum((double)kept);
    const int w = tid / kWave, l = tid % kWave;
    if (l == 0) {
        redd[w] = sum;
        redd[NT / kWave + w] = kd;
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0, kt = 0.0;
#pragma unroll
        for (int i = 0; i < NT / kWave; ++i) {
            tot += redd[i];
            kt += redd[NT / kWave + i];
        }
        RowPartial rp;
        rp.m = m;
        rp.nkept = (int)kt;
        rp.s = m == -INFINITY ? 0.0 : tot * exp2(-(double)emc);
        a.part[row] = rp;
        a.row_thr[row] = thr;
    }
}

// ---------------------------------------------------------------------------------------
// Decision and sampling, in three launches with kernel boundaries as the only
// synchronization:
//   1. decision: one workgroup per request combines its rows' partials in fp64, evaluates
//      p_i(y_i), q_i(y_i) and the accept test left to right, finds the first rejection and
//      publishes the accepted tokens;
//   2. chunk sums: one workgroup per (request, 8192-token chunk) of the row pair (or bonus
//      row) still to be sampled writes the chunk's four sub-chunk sums of the weights;
//   3. pick: one workgroup per request forms W from the sub-chunk sums, locates the
//      sub-chunk holding t = u * W and scans it in ascending token order for the smallest x
//      with C(x) > t. A residual whose mass comes out below kPreciseBelow is re-derived
//      there first with the precise arithmetic (precise_draw).
// Rows after the first rejection are never read.
// ---------------------------------------------------------------------------------------
constexpr int kDecideNT = 256;             // threads of a decision workgroup (>= 2*64+1 rows)
constexpr int kPartNT = 256;               // threads of a chunk-sum workgroup
constexpr int kPickNT = 256;               // threads of a pick workgroup
constexpr int kSChunk = 8192;              // tokens per sampling chunk
constexpr int kSSub = 4;                   // weight sums per chunk, one per sub-chunk
constexpr int kSSubLen = kSChunk / kSSub;  // tokens per sub-chunk
constexpr int kSMaxChunks = 256;           // V <= kSChunk * kSMaxChunks
static_assert(kSChunk * kSMaxChunks == SPECDEC_MAX_V, "sampling chunks cover the largest V");

struct Decision {
    int flags, err, a, k, mode, row_t, row_d;
    float T;                 // the request's temperature
    float mc_t, mc_d, thr_t, thr_d;
    double al_t, al_d;
    float u;
    float c;                 // log2(e) / T of the request
    float mt, md;            // max kept logit of the target / draft row of the draw
};

struct SampleArgs {
    const uint8_t* tgt;
    const uint8_t* dft;
    const int* tokens;
    const int* cu;
    const float* u_acc;
    const float* u_smp;
    int B, K, max_k, V;
    int nparts;              // statistics partials per row
    int topk;                // 1 when rows carry a top-k threshold
    int nch;                 // sampling chunks per row
    float c;
    float T;                 // the scalar temperature (per-request arrays: temps)
    const float* temps;      // [B] per-request temperatures, or null
    const RowParams* rpar;   // per-request parameters: [rows] each row's, else null
    const RowPartial* part;
    const float* row_thr;
    Decision* rec;           // [B] each request's decision, for the draw
    double* wsum;            // [B][nch][kSSub] sub-chunk sums of the sampling weights
    const int* kn;           // bf16 top-k: [K+B] kept tokens listed per target row, or null
    const uint32_t* ktok;    // [K+B][kKeptCap] kept tokens, ascending
    const uint16_t* kkey;    // [K+B][kKeptCap] their keys
    int* out_tokens;
    int* num_acc;
    int* num_emit;
    int* err_word;
    specdec_debug dbg;
    Decision* prec;          // analytics: [K] the row pair of every proposal position, else null
    double* wacc;            // analytics: [K][nch][kSSub] sub-chunk sums of max(0, p - q)
    const int* eos;          // [B] end-of-sequence token per request (< 0 none), or null
    const int* cap;          // [B] most tokens a request may emit (<= 0 none), or null
    int early;               // 1: rows past each request's first rejection were not read
    int* live;               // early exit: [2][B] each request's liveness, one buffer per
                             // launch parity
};

constexpr int kMaxRows = 2 * SPECDEC_MAX_K + 1;

// A row's max m and exp-sum S (and kept count) from its chunk partials, combined in fp64 in
// a fixed order: batches of eight, what was summed so far rescaled to the running max.
SD_DEV void combine_partials(const RowPartial* pp, int nparts, double cd, float* m_out,
                             double* S_out, int* nk_out) {
    float m = -INFINITY;
    double S = 0.0;
    int nk = 0;
    for (int q0 = 0; q0 < nparts; q0 += 8) {
        RowPartial x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {                // the batch's loads issue together
            if (q0 + q < nparts) x[q] = pp[q0 + q];
            else x[q] = RowPartial{-INFINITY, 0, 0.0};
        }
        float mb = -INFINITY;
#pragma unroll
        for (int q = 0; q < 8; ++q) mb = fmaxf(mb, x[q].m);
        const float mn = fmaxf(m, mb);
        if (m != -INFINITY && mn != m) S *= exp2((double)(m - mn) * cd);
        m = mn;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // chunks with no finite entry carry 0 (or NaN, which must propagate)
            S += x[q].m == -INFINITY ? x[q].s : x[q].s * exp2((double)(x[q].m - m) * cd);
            nk += x[q].nkept;
        }
    }
    *m_out = m;
    *S_out = S;
    *nk_out = nk;
}

// p(x) of a logit z in a row with max m, exp-sum S and threshold thr, in fp64
SD_DEV double kept_prob(float z, float m, double S, float thr, double cd) {
    return (z >= thr && z > -INFINITY) ? exp2(((double)z - (double)m) * cd) / S : 0.0;
}

// Weight of token x for the draw: max(0, p(x) - q(x)) after a rejection (RESID), p(x)
// for the bonus; p and q from fp32 exponentials of the form the statistics used, scaled
// by the rows' normalizers, in fp32 (about 2e-7 relative to p; a residual mass this path
// cannot resolve goes to the precise draw). TOPK masks tokens below the rows' thresholds.
template <bool RESID, bool TOPK>
SD_DEV float weight_t(float zt, float zd, const Decision& r, float c) {
    float pt = __builtin_amdgcn_exp2f(fmaf(zt, c, -r.mc_t)) * (float)r.al_t;
    if (TOPK && !(zt >= r.thr_t)) pt = 0.f;
    if (!RESID) return pt;
    float pd = __builtin_amdgcn_exp2f(fmaf(zd, c, -r.mc_d)) * (float)r.al_d;
    if (TOPK && !(zd >= r.thr_d)) pd = 0.f;
    return fmaxf(pt - pd, 0.f);
}

SD_DEV float weight(float zt, float zd, const Decision& r, float c, bool resid) {
    if (resid) return weight_t<true, true>(zt, zd, r, c);
    return weight_t<false, true>(zt, zd, r, c);
}

// Eight consecutive elements starting at i0 (a multiple of 8); -inf at or past V. FULL
// promises i0 + 8 <= V (no bounds test).
template <bool BF16, bool VEC, bool FULL = false>
SD_DEV void load8(const uint8_t* __restrict__ row, int V, int i0, float (&z)[8]) {
    if constexpr (VEC && BF16) {
        if (FULL || i0 < V) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + i0 / 8);
            const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                z[2 * j] = bf16_lo(q[j]);
                z[2 * j + 1] = bf16_hi(q[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) z[j] = -INFINITY;
        }
    } else if constexpr (VEC) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (FULL || i0 + 4 * h < V) {
                const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + i0 / 4 + h);
                z[4 * h] = __uint_as_float(w.x);
                z[4 * h + 1] = __uint_as_float(w.y);
                z[4 * h + 2] = __uint_as_float(w.z);
                z[4 * h + 3] = __uint_as_float(w.w);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) z[4 * h + j] = -INFINITY;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = (FULL || i0 + j < V) ? load_elem(row, i0 + j, BF16) : -INFINITY;
    }
}

// Decision of request b, computed by one workgroup of NT threads (all threads call): the
// row partials are combined in fp64, p_i(y_i) and q_i(y_i) evaluated in fp64, proposals
// accepted left to right while u * q < p. The result lands in D (LDS). With `publish` the
// workgroup also writes num_accepted / num_emitted, the accepted tokens, the error word
// and the diagnostics.
template <bool BF16, int NT>
SD_DEV void decide_body(const SampleArgs& a, int b, bool publish, Decision& D) {
    using Lt = Layout<BF16, true>;
    __shared__ float s_m[kMaxRows];
    __shared__ double s_S[kMaxRows];
    __shared__ float s_thr[kMaxRows];
    __shared__ int s_rowbad;
    __shared__ int s_bad[kMaxRows];     // early exit: each row's validity
    __shared__ int s_nk[kMaxRows];      // early exit: each row's kept count
    __shared__ int s_vis;               // early exit: the last visited position
    const int tid = threadIdx.x, lane = tid % kWave;
    const int rows_t = a.K + a.B;

    const int lo = a.cu[b], hi = a.cu[b + 1];
    const int k = hi - lo;
    const bool bad_k = a.cu[0] != 0 || a.cu[a.B] != a.K || k < 0 || k > a.max_k || lo < 0 ||
                       hi > a.K;
    if (bad_k) {
        if (tid == 0) {
            D.mode = MODE_NONE;
            D.flags = SPECDEC_ERR_K;
            if (publish) {
                a.num_acc[b] = -1;
                a.num_emit[b] = 0;
                atomicOr(a.err_word, SPECDEC_ERR_K);
                if (a.dbg.req_flags) a.dbg.req_flags[b] = SPECDEC_ERR_K;
            }
        }
        __syncthreads();
        return;
    }
    // the request's temperature (and whether its parameters are valid)
    float cf = a.c;
    int pbad = 0;
    if (a.rpar) {
        const RowParams rq = a.rpar[lo + b];
        cf = rq.c;
        pbad = rq.flags & kRpBad;
    }
    const double cd = (double)cf;
    if (tid == 0) s_rowbad = 0;
    __syncthreads();
    const int nrows = 2 * k + 1;   // <= kMaxRows <= NT
    if (tid < nrows) {
        const int r = tid;
        const int prow = r <= k ? lo + b + r : rows_t + lo + (r - k - 1);
        float m;
        double S;
        int nk;
        combine_partials(a.part + (size_t)prow * a.nparts, a.nparts, cd, &m, &S, &nk);
        const float thr = a.topk ? a.row_thr[prow] : -INFINITY;
        s_m[r] = m;
        s_S[r] = S;
        s_thr[r] = thr;
        const bool rbad = !(S > 0.0 && S < INFINITY && m > -INFINITY);
        if (a.early) {
            s_bad[r] = rbad;
            s_nk[r] = a.topk ? nk : -1;
        } else if (rbad) {
            atomicOr(&s_rowbad, 1);
        }
        if (publish && !a.early) {
            if (a.dbg.row_max) a.dbg.row_max[prow] = m;
            if (a.dbg.row_sum) a.dbg.row_sum[prow] = S;
            if (a.dbg.row_thr) a.dbg.row_thr[prow] = thr;
            if (a.dbg.row_nkept) a.dbg.row_nkept[prow] = a.topk ? nk : -1;
        }
    }
    __syncthreads();
    if (tid < kWave) {
        // lane i: proposal i (k <= SPECDEC_MAX_K = kWave)
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
                const float zt = load_elem(a.tgt + (size_t)(lo + b + lane) * a.V * Lt::ES, y, BF16);
                const float zd = load_elem(a.dft + (size_t)(lo + lane) * a.V * Lt::ES, y, BF16);
                const int rt = lane, rd = k + 1 + lane;
                P = kept_prob(zt, s_m[rt], s_S[rt], s_thr[rt], cd);
                Q = kept_prob(zd, s_m[rd], s_S[rd], s_thr[rd], cd);
                acc = u * Q < P;
            }
        }
        // early exit: the rows of position i were read only if proposals 0..i-1 passed the
        // test the statistics launches apply (valid uniform and token, accepted); the
        // request's visited positions are 0..vis
        bool rowbad = s_rowbad != 0;
        if (a.early) {
            const bool ok = (flags & (SPECDEC_ERR_UNIFORM | SPECDEC_ERR_TOKEN)) == 0 && acc;
            const unsigned long long stop = __ballot(lane < k && !ok);
            // invalid parameters: the statistics launches read none of the rows
            const int vis = pbad ? -1 : (stop ? (__ffsll((long long)stop) - 1) : k);
            int rb = 0;
            for (int r = lane; r < nrows; r += kWave)     // target rows 0..k, then draft rows
                if ((r <= k ? r : r - k - 1) <= vis) rb |= s_bad[r];
            rowbad = __ballot(rb) != 0ull;
            if (lane == 0) s_vis = vis;
            if (lane > vis && lane < k) P = Q = NAN;    // rows never read
        }
        const double us = (double)a.u_smp[b];
        if (lane == 0 && !(us >= 0.0 && us < 1.0)) flags |= SPECDEC_ERR_UNIFORM;
        if (lane == 0 && rowbad && !pbad) flags |= SPECDEC_ERR_NONFINITE;
        if (lane == 0 && pbad) flags |= SPECDEC_ERR_PARAM;
        const unsigned long long rej = __ballot(lane < k && !acc);
        const int j = rej ? (__ffsll((long long)rej) - 1) : k;
        if (lane < k && lane <= j && Q == 0.0 && !(flags & SPECDEC_ERR_TOKEN) && !pbad)
            flags |= SPECDEC_ERR_QZERO;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) flags |= __shfl_xor(flags, o, kWave);
        const bool err = (flags & (SPECDEC_ERR_TOKEN | SPECDEC_ERR_UNIFORM | SPECDEC_ERR_NONFINITE |
                                   SPECDEC_ERR_PARAM)) != 0;
        // stopping: the output ends at the first accepted EOS (inclusive) or at the cap,
        // when that falls within the accepted proposals; then nothing is drawn
        int L = j + 1;
        if (a.eos) {
            const int eos = a.eos[b];
            const unsigned long long hit = __ballot(lane < j && eos >= 0 && y == eos);
            if (hit) L = __ffsll((long long)hit);
        }
        if (a.cap) {
            const int cap = a.cap[b];
            if (cap > 0 && cap < L) L = cap;
        }
        const bool stop = L <= j;
        const int acc_n = stop ? L : j;            // proposals kept
        if (publish) {
            if (lane < k) {
                if (a.dbg.p_y) a.dbg.p_y[lo + lane] = P;
                if (a.dbg.q_y) a.dbg.q_y[lo + lane] = Q;
            }
            if (!err && lane < acc_n) a.out_tokens[lo + b + lane] = y;
            if (lane == 0) {
                a.num_acc[b] = err ? -1 : acc_n;
                a.num_emit[b] = err ? 0 : (stop ? L : j + 1);
                if (flags) atomicOr(a.err_word, flags);
                if (a.dbg.req_flags) a.dbg.req_flags[b] = flags;
            }
        }
        if (lane == 0) {
            Decision d;
            d.flags = flags;
            d.err = err;
            d.a = j;
            d.k = k;
            d.T = a.temps ? a.temps[b] : a.T;
            d.c = cf;
            d.mode = (err || stop) ? MODE_NONE : (j < k ? MODE_RESID : MODE_BONUS);
            d.row_t = lo + b + j;
            d.row_d = j < k ? lo + j : 0;
            const float mt = s_m[j];
            d.mt = mt;
            d.md = j < k ? s_m[k + 1 + j] : 0.f;
            d.mc_t = mt * cf;
            d.al_t = exp2(-(double)fmaf(mt, cf, -d.mc_t)) / s_S[j];
            d.thr_t = s_thr[j];
            if (j < k) {
                const float md = s_m[k + 1 + j];
                d.mc_d = md * cf;
                d.al_d = exp2(-(double)fmaf(md, cf, -d.mc_d)) / s_S[k + 1 + j];
                d.thr_d = s_thr[k + 1 + j];
            } else {
                d.mc_d = 0.f;
                d.al_d = 0.0;
                d.thr_d = INFINITY;
            }
            d.u = a.u_smp[b];
            D = d;
        }
        if (publish && a.prec && lane < k) {
            // analytics: the row pair of this position, for the residual mass of every one
            Decision q;
            q.flags = 0;
            q.err = err;
            q.a = lane;
            q.k = k;
            q.mode = err ? MODE_NONE : MODE_RESID;
            q.row_t = lo + b + lane;
            q.row_d = lo + lane;
            q.T = a.temps ? a.temps[b] : a.T;
            q.c = cf;
            q.u = 0.f;
            const float mt = s_m[lane], md = s_m[k + 1 + lane];
            q.mt = mt;
            q.md = md;
            q.mc_t = mt * cf;
            q.al_t = exp2(-(double)fmaf(mt, cf, -q.mc_t)) / s_S[lane];
            q.thr_t = s_thr[lane];
            q.mc_d = md * cf;
            q.al_d = exp2(-(double)fmaf(md, cf, -q.mc_d)) / s_S[k + 1 + lane];
            q.thr_d = s_thr[k + 1 + lane];
            a.prec[lo + lane] = q;
        }
    }
    __syncthreads();
    if (a.early && publish && tid < nrows) {
        // early exit: statistics of the visited rows; rows never read report NaN
        const int prow = tid <= k ? lo + b + tid : rows_t + lo + (tid - k - 1);
        const bool seen = (tid <= k ? tid : tid - k - 1) <= s_vis;
        if (a.dbg.row_max) a.dbg.row_max[prow] = seen ? s_m[tid] : NAN;
        if (a.dbg.row_sum) a.dbg.row_sum[prow] = seen ? s_S[tid] : NAN;
        if (a.dbg.row_thr) a.dbg.row_thr[prow] = seen ? s_thr[tid] : NAN;
        if (a.dbg.row_nkept) a.dbg.row_nkept[prow] = seen ? s_nk[tid] : -1;
    }
}

// Sums of the sampling weights over the kSSub sub-chunks (kSSubLen consecutive tokens
// each) of one chunk of the row (pair) still to be sampled, by a workgroup of NT threads:
// group g of every thread lies in sub-chunk g, and all of them are in flight at once.
// Fixed reduction order (lanes, then waves in index order). Thread s < kSSub writes
// out[s]; `red` holds kSSub * NT / 64 doubles.
template <bool BF16, bool VEC, int NT, bool RESID, bool TOPK>
SD_DEV void chunk_weight_sums_t(const uint8_t* trow, const uint8_t* drow, int V, int chunk,
                                const Decision& r, float c, double* red, double* out) {
    constexpr int NW = NT / kWave;
    static_assert(NT * 8 * kSSub == kSChunk, "group g of every thread is sub-chunk g");
    const int tid = threadIdx.x;
    const int w = tid / kWave, l = tid % kWave;
    if constexpr (BF16 && VEC) {
        // packed bf16 stays packed until used: fewer registers, more workgroups per CU
        const u32x4* tv = reinterpret_cast<const u32x4*>(trow);
        const u32x4* dv = reinterpret_cast<const u32x4*>(drow);
        const u32x4 ninf = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
        u32x4 rt[kSSub], rd[kSSub];
        const bool full = (chunk + 1) * kSChunk <= V;
#pragma unroll
        for (int g = 0; g < kSSub; ++g) {
            const int i0 = chunk * kSChunk + (g * NT + tid) * 8;
            rt[g] = full || i0 < V ? __builtin_nontemporal_load(tv + i0 / 8) : ninf;
            if (RESID) rd[g] = full || i0 < V ? __builtin_nontemporal_load(dv + i0 / 8) : ninf;
        }
#pragma unroll
        for (int g = 0; g < kSSub; ++g) {
            const uint32_t qt[4] = {rt[g].x, rt[g].y, rt[g].z, rt[g].w};
            uint32_t qd[4] = {0u, 0u, 0u, 0u};
            if (RESID) {
                qd[0] = rd[g].x;
                qd[1] = rd[g].y;
                qd[2] = rd[g].z;
                qd[3] = rd[g].w;
            }
            float acc = 0.f;               // the thread's 8 weights in fp32, in order
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc += weight_t<RESID, TOPK>(bf16_lo(qt[j]), bf16_lo(qd[j]), r, c);
                acc += weight_t<RESID, TOPK>(bf16_hi(qt[j]), bf16_hi(qd[j]), r, c);
            }
            const double sum = wave_sum((double)acc);
            if (l == 0) red[g * NW + w] = sum;
        }
    } else {
        float zt[kSSub][8], zd[kSSub][8];
        if ((chunk + 1) * kSChunk <= V) {          // whole chunk inside the row
#pragma unroll
            for (int g = 0; g < kSSub; ++g) {
                const int i0 = chunk * kSChunk + (g * NT + tid) * 8;
                load8<BF16, VEC, true>(trow, V, i0, zt[g]);
                if (RESID) load8<BF16, VEC, true>(drow, V, i0, zd[g]);
            }
        } else {
#pragma unroll
            for (int g = 0; g < kSSub; ++g) {
                const int i0 = chunk * kSChunk + (g * NT + tid) * 8;
                load8<BF16, VEC>(trow, V, i0, zt[g]);
                if (RESID) load8<BF16, VEC>(drow, V, i0, zd[g]);
            }
        }
#pragma unroll
        for (int g = 0; g < kSSub; ++g) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += weight_t<RESID, TOPK>(zt[g][e], zd[g][e], r, c);
            const double sum = wave_sum((double)acc);
            if (l == 0) red[g * NW + w] = sum;
        }
    }
    __syncthreads();
    if (tid < kSSub) {
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < NW; ++i) sum += red[tid * NW + i];
        out[tid] = sum;
    }
    __syncthreads();
}

template <bool BF16, bool VEC, int NT>
SD_DEV void chunk_weight_sums(const uint8_t* trow, const uint8_t* drow, int V, int chunk,
                              const Decision& r, float c, bool resid, bool topk, double* red,
                              double* out) {
    if (resid) {
        if (topk) chunk_weight_sums_t<BF16, VEC, NT, true, true>(trow, drow, V, chunk, r, c, red, out);
        else chunk_weight_sums_t<BF16, VEC, NT, true, false>(trow, drow, V, chunk, r, c, red, out);
    } else {
        if (topk) chunk_weight_sums_t<BF16, VEC, NT, false, true>(trow, drow, V, chunk, r, c, red, out);
        else chunk_weight_sums_t<BF16, VEC, NT, false, false>(trow, drow, V, chunk, r, c, red, out);
    }
}

// Decision kernel body: one workgroup per request publishes its decision and stores it
// for the sampling workgroups.
template <bool BF16, int NT>
SD_DEV void decide_kernel_body(const SampleArgs& a, int b) {
    __shared__ Decision D;
    decide_body<BF16, NT>(a, b, true, D);
    if (threadIdx.x == 0) a.rec[b] = D;
}

// ---------------------------------------------------------------------------------------
// Early exit (an opt-in cycle): the statistics of the first positions run one launch per
// position, then one more launch reads every remaining row of each request still live.
// Workgroup (b, side, chunk) of position launch p reads its chunk of request b's target
// row p (side 0) or draft row p (side 1, only while p < k_b) if every proposal before p
// passed the accept test with a valid uniform and token. That test is evaluated again here
// from the partials the earlier launches wrote, with the decision's own arithmetic
// (combine_partials, kept_prob, u * Q < P), so both agree on the rows that were read. The
// last launch (tail_body) does the same test at its position and then reads the chunk of
// every later row of the request, ahead of knowing whether the decision needs them: one
// launch instead of one per position, for the few requests still live. No row past a
// rejection at an earlier position is read; the decision, the draw and the cache steps
// then run as in the full cycle. Temperature only, scalar or per request (no top-k /
// top-p): partials are per chunk.
// ---------------------------------------------------------------------------------------

// positions 0 .. kEarlyCut - 1 one launch each, then one launch for every later row of the
// requests still live
constexpr int kEarlyCut = SPECDEC_EARLY_EXIT_SEQUENTIAL;
static_assert(kEarlyCut >= 1, "position 0 is read for every request first");
// rows from position p on of a request with k_b <= max_k: target rows p .. k_b and draft
// rows p .. k_b - 1, at most 2 (max_k - p) + 1
__host__ __device__ inline int early_tail_slots(int max_k, int p) { return 2 * (max_k - p) + 1; }

// Whether request b (first proposal lo, k_b = k) is live at position p >= 1, given that it
// was live at p - 1 (the flag the launch for p - 1 left) and p <= k: proposal p - 1 has a
// valid uniform and token and passes u * Q < P, with P and Q formed as the decision forms
// them (the rows' combined partials, and their thresholds when a top-k / top-p transform
// is on). Threads 0 and 1 of the workgroup call: thread 0 evaluates the target row, thread
// 1 the draft row; thread 0's result counts.
template <bool BF16>
SD_DEV bool live_test(const SampleArgs& a, const RowPartial* part, int p, int b, int lo) {
    using Lt = Layout<BF16, true>;
    const int lane = threadIdx.x;
    const int nchunks = a.nparts;
    const int rows_t = a.K + a.B;
    const int i = lo + p - 1;
    const int y = a.tokens[i];
    const double u = (double)a.u_acc[i];
    bool live = u >= 0.0 && u < 1.0 && y >= 0 && y < a.V;
    if (live) {
        // the request's log2(e) / T, as the decision takes it
        const double cd = (double)(a.rpar ? a.rpar[lo + b].c : a.c);
        const size_t prow = lane == 0 ? (size_t)(i + b) : (size_t)(rows_t + i);
        const uint8_t* zrow = lane == 0 ? a.tgt + (size_t)(i + b) * a.V * Lt::ES
                                        : a.dft + (size_t)i * a.V * Lt::ES;
        float m;
        double S;
        int nk;
        combine_partials(part + prow * nchunks, nchunks, cd, &m, &S, &nk);
        const float thr = a.topk ? a.row_thr[prow] : -INFINITY;
        const double pr = kept_prob(load_elem(zrow, y, BF16), m, S, thr, cd);
        const double Q = __shfl(pr, 1, kWave);
        live = u * Q < pr;                           // lane 0's: P = its own
    }
    return live;
}

// The early-exit grids. pass_grid: workgroup w of a (request, side, chunk) grid at
// position p; the liveness chain (p = 0: the request's offsets and parameters are valid;
// p >= 1: live at p - 1 and proposal p - 1 accepted), the flag for the next launch, then
// work(row, chunk) for the row of this side at p if the request is live and has it.
// tail_grid: if the request is live at p >= 1, work(row, chunk) for its target rows
// p .. k_b and draft rows p .. k_b - 1, and (with `flag`) the liveness at p left for a
// later launch. SLOTS: workgroup w of a (request, row slot, chunk) grid with
// early_tail_slots(max_k, p) slots per request (slots 0 .. k_b - p the target rows, the
// slots after them the draft rows), one row each: the chunk select, several times the
// work of the plain statistics, keeps the few live requests' rows side by side; else
// workgroup w of a (request, chunk) grid takes the chunk of every row in turn, which for
// the plain statistics costs less than one liveness test per row. nchunks: the grid's
// chunks per row.
template <bool BF16, class Work>
SD_DEV void pass_grid(const SampleArgs& a, int nchunks, int p, int w, Work&& work) {
    __shared__ int s_live;
    const int b = w / (2 * nchunks);
    const int side = (w / nchunks) & 1;
    const int chunk = w - (w / nchunks) * nchunks;
    const int rows_t = a.K + a.B;
    const int lo = a.cu[b], hi = a.cu[b + 1];
    const int k = hi - lo;
    if (p > 0 && (a.live[((p - 1) & 1) * a.B + b] == 0 || p > k)) {
        // not live: every thread leaves at once (the flag is the same for the whole
        // workgroup); one workgroup per request passes the 0 on
        if (side == 0 && chunk == 0 && threadIdx.x == 0) a.live[(p & 1) * a.B + b] = 0;
        return;
    }
    if (threadIdx.x < 2) {
        bool live;
        if (p == 0) {
            live = !(a.cu[0] != 0 || a.cu[a.B] != a.K || k < 0 || k > a.max_k || lo < 0 ||
                     hi > a.K);
            // a request with invalid parameters fails in the decision without its rows
            if (live && a.rpar) live = !(a.rpar[lo + b].flags & kRpBad);
        } else {
            live = live_test<BF16>(a, a.part, p, b, lo);
        }
        if (threadIdx.x == 0) {
            // one workgroup per request leaves the flag for the next launch (every launch
            // writes every request's flag, so none is stale)
            if (side == 0 && chunk == 0) a.live[(p & 1) * a.B + b] = live ? 1 : 0;
            s_live = live && (side == 0 || p < k);
        }
    }
    __syncthreads();
    if (!s_live) return;
    work(side == 0 ? lo + b + p : rows_t + lo + p, chunk);
}

template <bool BF16, bool SLOTS, class Work>
SD_DEV void tail_grid(const SampleArgs& a, int nchunks, int p, int w, bool flag, Work&& work) {
    __shared__ int s_live;
    const int per = SLOTS ? early_tail_slots(a.max_k, p) : 1;
    const int chunk = w % nchunks;
    const int b = w / nchunks / per;
    const int j = w / nchunks - b * per;
    const int rows_t = a.K + a.B;
    const int lo = a.cu[b], hi = a.cu[b + 1];
    const int k = hi - lo;
    const bool first = j == 0 && chunk == 0;         // leaves the flag
    if (p > k || a.live[((p - 1) & 1) * a.B + b] == 0) {
        if (flag && first && threadIdx.x == 0) a.live[(p & 1) * a.B + b] = 0;
        return;
    }
    int row = 0;
    if (SLOTS) {
        if (j <= k - p) {
            row = lo + b + p + j;                      // target rows p .. k
        } else {
            const int i = p + (j - (k - p + 1));       // draft rows p .. k - 1
            row = i < k ? rows_t + lo + i : -1;
        }
        if (row < 0 && !(flag && first)) return;
    }
    if (threadIdx.x < 2) {
        const bool live = live_test<BF16>(a, a.part, p, b, lo);
        if (threadIdx.x == 0) {
            if (flag && first) a.live[(p & 1) * a.B + b] = live ? 1 : 0;
            s_live = live && row >= 0;
        }
    }
    __syncthreads();
    if (!s_live) return;
    if (SLOTS) {
        work(row, chunk);
    } else {
        for (int i = p; i <= k; ++i) {
            work(lo + b + i, chunk);
            if (i < k) work(rows_t + lo + i, chunk);
        }
    }
}

// Early exit with the plain statistics (temperature only): launch p reads position p's
// rows of the requests live at p; the last launch every later row of those still live.
template <bool BF16, bool VEC>
SD_DEV void pass_body(const SampleArgs& a, RowPartial* __restrict__ part, int p, int w) {
    const int nchunks = a.nparts;
    pass_grid<BF16>(a, nchunks, p, w, [&](int row, int chunk) {
        row_stats_body<BF16, VEC>(a.tgt, a.dft, a.K + a.B, a.V, nchunks, a.c, part,
                                  row * nchunks + chunk, a.rpar);
    });
}

template <bool BF16, bool VEC>
SD_DEV void tail_body(const SampleArgs& a, RowPartial* __restrict__ part, int p, int w) {
    const int nchunks = a.nparts;
    tail_grid<BF16, false>(a, nchunks, p, w, false, [&](int row, int chunk) {
        row_stats_body<BF16, VEC>(a.tgt, a.dft, a.K + a.B, a.V, nchunks, a.c, part,
                                  row * nchunks + chunk, a.rpar);
    });
}

// ---------------------------------------------------------------------------------------
// Precise residual draw. The streaming draw forms max(0, p - q) from fp32 exponentials of
// each row, normalized by each row's exp-sum, so the difference carries an absolute error
// of about 1e-7 of p: harmless while the residual mass W is large, not once W is small
// (close distributions) or zero (distributions that agree). A draw whose streaming mass
// comes out below kPreciseBelow is re-derived by its pick workgroup without that
// cancellation:
//   a(x)     = exp((z_t(x) - m_t) / T)                 target weight (fp32 exponential)
//   delta(x) = ((z_d(x) - m_d) - (z_t(x) - m_t)) / T   exact differences, one fp64 rounding
//   q(x) / p(x) = exp(delta(x) - lambda),   lambda = log(S_d / S_t)
//   S_d / S_t - 1 = (sum_both a expm1(delta) + sum_draft-only e_d - sum_target-only a) / A
//   w(x) = a(x) max(0, -expm1(delta(x) - lambda))      kept on both sides
//        = a(x)                                        kept by the target only
// with A the sum of a over the target's kept tokens and every sum in fp64. S_d / S_t is a
// weighted mean of exp(delta) under the same a values that weight the tokens, so an error
// in a(x) moves lambda only through the spread of delta, and rows that agree (equal kept
// sets, delta = 0 on every kept token) give lambda = 0 and w = 0 everywhere: W = 0 exactly,
// as the definition has it. Each weight then carries the relative error of a(x), about
// 1e-7, whatever the size of W.
// ---------------------------------------------------------------------------------------
constexpr double kPreciseBelow = 0.25;

struct PreciseRow {
    double mt, md;      // max kept logit of the target / draft row
    double invT;        // 1 / T
    double l2T;         // log2(e) / T, for the fp32 exponentials of the weights
    double lam;         // log(S_d / S_t)
    float thr_t, thr_d;
};

SD_DEV double precise_a(double dz, const PreciseRow& P) {
    return (double)__builtin_amdgcn_exp2f((float)(dz * P.l2T));
}

// Pass 1 terms of one token: A += a(x) for a kept target token, N += its share of
// S_d - S_t (in units of the target's max-normalized exp-sum).
SD_DEV void precise_terms(float zt, float zd, const PreciseRow& P, double& A, double& N) {
    const bool kt = zt >= P.thr_t && zt > -INFINITY;
    const bool kd = zd >= P.thr_d && zd > -INFINITY;
    const double dt = (double)zt - P.mt;
    if (kt) {
        const double a = precise_a(dt, P);
        A += a;
        N += kd ? a * expm1((((double)zd - P.md) - dt) * P.invT) : -a;
    } else if (kd) {
        N += precise_a((double)zd - P.md, P);
    }
}

// The precise draw's weight of one token: the residual (RESID) or p, both unnormalized
// (in units of A).
SD_DEV double precise_weight(float zt, float zd, const PreciseRow& P, bool resid) {
    if (!(zt >= P.thr_t && zt > -INFINITY)) return 0.0;
    const double dt = (double)zt - P.mt;
    const double a = precise_a(dt, P);
    if (!resid || !(zd >= P.thr_d && zd > -INFINITY)) return a;
    const double ell = (((double)zd - P.md) - dt) * P.invT - P.lam;
    return a * fmax(0.0, -expm1(ell));
}

// One chunk of the row pair, kSSub groups of 8 tokens per thread with every load in flight
// (group g of every thread lies in sub-chunk g, as in chunk_weight_sums_t).
template <bool BF16, bool VEC, int NT>
SD_DEV void precise_load(const uint8_t* trow, const uint8_t* drow, int V, int chunk, bool pair,
                         float (&zt)[kSSub][8], float (&zd)[kSSub][8]) {
    static_assert(NT * 8 * kSSub == kSChunk, "group g of every thread is sub-chunk g");
#pragma unroll
    for (int g = 0; g < kSSub; ++g) {
        const int i0 = chunk * kSChunk + (g * NT + threadIdx.x) * 8;
        load8<BF16, VEC>(trow, V, i0, zt[g]);
        if (pair) {
            load8<BF16, VEC>(drow, V, i0, zd[g]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) zd[g][e] = -INFINITY;
        }
    }
}

// Pass 1 over the row pair: A and lambda (every thread gets both). `red` holds NT / 64
// doubles.
template <bool BF16, bool VEC, int NT>
SD_DEV double precise_lambda(const uint8_t* trow, const uint8_t* drow, int V, int nch,
                             PreciseRow& P, double* red) {
    double A = 0.0, N = 0.0;
    for (int ch = 0; ch < nch; ++ch) {
        float zt[kSSub][8], zd[kSSub][8];
        precise_load<BF16, VEC, NT>(trow, drow, V, ch, true, zt, zd);
#pragma unroll
        for (int g = 0; g < kSSub; ++g) {
#pragma unroll
            for (int e = 0; e < 8; ++e) precise_terms(zt[g][e], zd[g][e], P, A, N);
        }
    }
    A = block_sum<NT>(A, red);
    N = block_sum<NT>(N, red);
    P.lam = log1p(N / A);
    return A;
}

// Pass 2: the sub-chunk sums of the precise weights into out[0 .. nch * kSSub), fixed
// reduction order (lanes, then waves in index order). `red` holds kSSub * NT / 64 doubles.
template <bool BF16, bool VEC, int NT>
SD_DEV void precise_sums(const uint8_t* trow, const uint8_t* drow, int V, int nch,
                         const PreciseRow& P, bool resid, double* red, double* out) {
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
    for (int ch = 0; ch < nch; ++ch) {
        float zt[kSSub][8], zd[kSSub][8];
        precise_load<BF16, VEC, NT>(trow, drow, V, ch, resid, zt, zd);
#pragma unroll
        for (int g = 0; g < kSSub; ++g) {
            double acc = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += precise_weight(zt[g][e], zd[g][e], P, resid);
            acc = wave_sum(acc);
            if (l == 0) red[g * NW + w] = acc;
        }
        __syncthreads();
        if (tid < kSSub) {
            double sum = 0.0;
#pragma unroll
            for (int i = 0; i < NW; ++i) sum += red[tid * NW + i];
            out[ch * kSSub + tid] = sum;
        }
        __syncthreads();
    }
}

// Draw from the target row's kept-token list (bf16 top-k rows). Tokens outside the list
// have p = 0 and so weight 0 in both the residual and the bonus draw, so scanning the list
// in ascending token order finds the same smallest x with C(x) > u * W as scanning the
// vocabulary; the weights are the streaming draw's, token by token. One workgroup of NT
// threads, kKeptCap / NT consecutive list entries per thread.
template <bool BF16, int NT>
SD_DEV void listed_pick_body(const SampleArgs& a, int b, Decision r, int n) {
    constexpr int EPT = kKeptCap / NT;
    static_assert(EPT * NT == kKeptCap, "whole list entries per thread");
    __shared__ double redd[NT / kWave];
    __shared__ int redi[NT / kWave];
    __shared__ double s_wpick;
    const int tid = threadIdx.x;
    const uint32_t* tok = a.ktok + (size_t)r.row_t * kKeptCap;
    const uint16_t* key = a.kkey + (size_t)r.row_t * kKeptCap;
    const uint8_t* drow = a.dft + (size_t)r.row_d * a.V * (BF16 ? 2 : 4);
    const bool resid = r.mode == MODE_RESID;
    int x[EPT];
    float zt[EPT], zd[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid * EPT + e;
        x[e] = -1;
        zt[e] = zd[e] = -INFINITY;
        if (i < n) {
            x[e] = (int)tok[i];
            zt[e] = key_to_float<BF16>(key[i]);
            if (resid) zd[e] = load_elem(drow, x[e], BF16);
        }
    }
    double w[EPT];
    double run = 0.0, W;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        w[e] = x[e] >= 0 ? weight(zt[e], zd[e], r, r.c, resid) : 0.0;
        run += w[e];
    }
    double C = block_excl_scan_d<NT>(run, redd, &W);
    if (resid && !(W >= kPreciseBelow)) {
        // a small (or zero) residual: the pick launch re-derives it with the precise
        // arithmetic over the whole row pair (the draft's kept tokens outside the list
        // enter its normalization)
        if (tid == 0) a.rec[b].mode = MODE_PRECISE;
        return;
    }
    const double t = (double)r.u * W;
    int mine = 0x7fffffff, lastpos = -1;
    double wmine = 0.0, wlast = 0.0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        if (x[e] < 0) continue;
        C += w[e];
        if (mine == 0x7fffffff && C > t) {
            mine = x[e];
            wmine = w[e];
        }
        if (w[e] > 0.0) {
            lastpos = x[e];
            wlast = w[e];
        }
    }
    int found = block_min_i<NT>(mine, redi);
    if (found != 0x7fffffff) {
        if (mine == found) s_wpick = wmine;
    } else {
        found = block_max_i<NT>(lastpos, redi);
        if (found >= 0 && lastpos == found) s_wpick = wlast;
    }
    __syncthreads();
    if (tid == 0) {
        a.out_tokens[a.cu[b] + b + r.a] = found;
        if (a.dbg.resid_mass) a.dbg.resid_mass[b] = W;
        if (a.dbg.picked_prob) a.dbg.picked_prob[b] = s_wpick / W;
        if (a.dbg.req_flags) a.dbg.req_flags[b] = r.flags;
    }
}

// Sampling, part 1: workgroup (b, chunk) writes the sub-chunk sums of the weights of the
// row (pair) b still has to sample. Rows after the first rejection are never read.
template <bool BF16, bool VEC, int NT>
SD_DEV void part_body(const SampleArgs& a, int b, int chunk) {
    using Lt = Layout<BF16, VEC>;
    __shared__ double red[kSSub * (NT / kWave)];
    const Decision r = a.rec[b];
    if (r.mode == MODE_NONE) return;
    if constexpr (BF16) {
        if (a.kn) {
            const int n = a.kn[r.row_t];
            if (n >= 0) {             // the whole draw from the kept-token list
                if (chunk == 0) listed_pick_body<BF16, NT>(a, b, r, n);
                return;
            }
        }
    }
    const bool resid = r.mode == MODE_RESID;
    const uint8_t* trow = a.tgt + (size_t)r.row_t * a.V * Lt::ES;
    const uint8_t* drow = a.dft + (size_t)r.row_d * a.V * Lt::ES;
    chunk_weight_sums<BF16, VEC, NT>(trow, drow, a.V, chunk, r, r.c, resid, a.topk != 0, red,
                                     a.wsum + ((size_t)b * a.nch + chunk) * kSSub);
}

// The sub-chunk sums s[0 .. n) of a draw (n <= 4 * NT, thread i owning entries 4i .. 4i+3):
// their total W, then the sub-chunk q holding t = u * W, the first whose running sum
// through it exceeds t (the last non-empty one if rounding leaves none), and the running
// sum before it. Fixed association order; every thread gets the results. `red` holds
// NT / 64 doubles, `redi` NT / 64 ints.
template <int NT>
SD_DEV double subchunk_total(const double* s, int n, double* red) {
    double v = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = threadIdx.x * 4 + j;
        if (q < n) v += s[q];
    }
    return block_sum<NT>(v, red);
}

template <int NT>
SD_DEV int subchunk_locate(const double* s, int n, double t, double* red, int* redi,
                           double* base_out) {
    __shared__ double s_base;
    double v[4], run = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = threadIdx.x * 4 + j;
        v[j] = q < n ? s[q] : 0.0;
        run += v[j];
    }
    double tot;
    double C = block_excl_scan_d<NT>(run, red, &tot);
    int mine = 0x7fffffff, lastpos = -1;
    double cmine = 0.0, clast = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = threadIdx.x * 4 + j;
        if (mine == 0x7fffffff && C + v[j] > t) {
            mine = q;
            cmine = C;
        }
        if (v[j] > 0.0) {
            lastpos = q;
            clast = C;
        }
        C += v[j];
    }
    int q = block_min_i<NT>(mine, redi);
    if (q != 0x7fffffff) {
        if (mine == q) s_base = cmine;
    } else {
        q = block_max_i<NT>(lastpos, redi);
        if (q < 0) {
            q = 0;
            if (threadIdx.x == 0) s_base = 0.0;
        } else if (lastpos == q) {
            s_base = clast;
        }
    }
    __syncthreads();
    *base_out = s_base;
    __syncthreads();
    return q;
}

// Sampling, part 2: workgroup b turns the sub-chunk sums into W, finds the sub-chunk holding
// t = u * W and scans it in ascending token order (each thread owns 8 consecutive tokens,
// an exclusive scan over threads gives each its running sum) for the smallest x with
// C(x) > t. A residual of streaming mass below kPreciseBelow (or one the kept-token list
// handed over as MODE_PRECISE) is re-derived first with the precise arithmetic; a precise
// residual of mass 0 falls back to p (flagged).
template <bool BF16, bool VEC, int NT>
SD_DEV void pick_body(const SampleArgs& a, int b) {
    using Lt = Layout<BF16, VEC>;
    constexpr int NW = NT / kWave;
    static_assert(NT * 8 == kSSubLen, "8 tokens per thread cover a sub-chunk");
    __shared__ double red[kSSub * NW];
    __shared__ int redi[NW];
    __shared__ double s_cs[kSMaxChunks * kSSub];
    __shared__ double s_wpick;
    const int tid = threadIdx.x;
    Decision r = a.rec[b];
    if (r.mode == MODE_NONE) return;
    if constexpr (BF16) {
        // drawn from the kept-token list, unless the list handed the draw over
        if (r.mode != MODE_PRECISE && a.kn && a.kn[r.row_t] >= 0) return;
    }
    bool resid = r.mode != MODE_BONUS;
    const uint8_t* trow = a.tgt + (size_t)r.row_t * a.V * Lt::ES;
    const uint8_t* drow = a.dft + (size_t)r.row_d * a.V * Lt::ES;
    const int nch = a.nch, nsub = nch * kSSub;
    static_assert(kSMaxChunks * kSSub <= 4 * NT, "four sub-chunk sums per thread");
    bool precise = r.mode == MODE_PRECISE;
    double W = 0.0;
    if (!precise) {
        for (int q = tid; q < nsub; q += NT) s_cs[q] = a.wsum[(size_t)b * nsub + q];
        __syncthreads();
        W = subchunk_total<NT>(s_cs, nsub, red);
        precise = resid && !(W >= kPreciseBelow);
    }
    PreciseRow P;
    double wscale = 1.0;      // reported W = the sum of the weights times wscale
    if (precise) {
        P.mt = (double)r.mt;
        P.md = (double)r.md;
        P.invT = 1.0 / (double)r.T;
        P.l2T = 1.4426950408889634074 * P.invT;
        P.thr_t = r.thr_t;
        P.thr_d = r.thr_d;
        P.lam = 0.0;
        const double A = precise_lambda<BF16, VEC, NT>(trow, drow, a.V, nch, P, red);
        wscale = 1.0 / A;
        precise_sums<BF16, VEC, NT>(trow, drow, a.V, nch, P, true, red, s_cs);
        W = subchunk_total<NT>(s_cs, nsub, red);
        if (!(W > 0.0)) {
            // the rows agree: no residual mass, draw the replacement from p_j instead
            resid = false;
            r.flags |= SPECDEC_ERR_ZFALLBACK;
            precise_sums<BF16, VEC, NT>(trow, drow, a.V, nch, P, false, red, s_cs);
            W = subchunk_total<NT>(s_cs, nsub, red);
            if (tid == 0) atomicOr(a.err_word, SPECDEC_ERR_ZFALLBACK);
        }
    }
    const double t = (double)r.u * W;
    double base;
    const int sub = subchunk_locate<NT>(s_cs, nsub, t, red, redi, &base);
    const int i0 = sub * kSSubLen + tid * 8;
    float t8[8], d8[8];
    load8<BF16, VEC>(trow, a.V, i0, t8);
    if (resid) load8<BF16, VEC>(drow, a.V, i0, d8);
    double w[8];
    double run = 0.0;
    if (precise) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            w[e] = precise_weight(t8[e], resid ? d8[e] : -INFINITY, P, resid);
            run += w[e];
        }
    } else {
        float run32 = 0.f;         // the thread's 8 weights as the chunk sums added them
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float wf = weight(t8[e], resid ? d8[e] : -INFINITY, r, r.c, resid);
            w[e] = (double)wf;
            run32 += wf;
        }
        run = (double)run32;
    }
    double tot;
    double C = base + block_excl_scan_d<NT>(run, red, &tot);
    int mine = 0x7fffffff, lastpos = -1;
    double wmine = 0.0, wlast = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        C += w[e];
        if (mine == 0x7fffffff && C > t) {
            mine = i0 + e;
            wmine = w[e];
        }
        if (w[e] > 0.0) {
            lastpos = i0 + e;
            wlast = w[e];
        }
    }
    int found = block_min_i<NT>(mine, redi);
    if (found != 0x7fffffff) {
        if (mine == found) s_wpick = wmine;
    } else {
        found = block_max_i<NT>(lastpos, redi);
        if (found >= 0 && lastpos == found) s_wpick = wlast;
    }
    __syncthreads();
    if (tid == 0) {
        a.out_tokens[a.cu[b] + b + r.a] = found;
        if (a.dbg.resid_mass) a.dbg.resid_mass[b] = W * wscale;
        if (a.dbg.picked_prob) a.dbg.picked_prob[b] = s_wpick / W;
        if (a.dbg.req_flags) a.dbg.req_flags[b] = r.flags;
    }
}

// ---------------------------------------------------------------------------------------
// Acceptance analytics: beta_i = 1 - W_i for every proposal position, W_i the residual mass
// sum_x max(0, p_i(x) - q_i(x)) summed exactly as the draw sums it; E[A] per request.
// ---------------------------------------------------------------------------------------
// W over a bf16 target row's kept-token list (tokens outside it have p = 0).
template <bool BF16, int NT>
SD_DEV double listed_resid_sum(const SampleArgs& a, const Decision& q, int n) {
    constexpr int EPT = kKeptCap / NT;
    __shared__ double redd[NT / kWave];
    const int tid = threadIdx.x;
    const uint32_t* tok = a.ktok + (size_t)q.row_t * kKeptCap;
    const uint16_t* key = a.kkey + (size_t)q.row_t * kKeptCap;
    const uint8_t* drow = a.dft + (size_t)q.row_d * a.V * (BF16 ? 2 : 4);
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid * EPT + e;
        if (i < n) {
            const int x = (int)tok[i];
            run += weight(key_to_float<BF16>(key[i]), load_elem(drow, x, BF16), q, q.c, true);
        }
    }
    return block_sum<NT>(run, redd);
}

// Workgroup (position r, chunk): the chunk's four sub-chunk sums of max(0, p - q).
template <bool BF16, bool VEC, int NT>
SD_DEV void accept_part_body(const SampleArgs& a, int r, int chunk) {
    using Lt = Layout<BF16, VEC>;
    __shared__ double red[kSSub * (NT / kWave)];
    const Decision q = a.prec[r];
    if (q.mode == MODE_NONE) return;
    double* out = a.wacc + ((size_t)r * a.nch + chunk) * kSSub;
    if constexpr (BF16) {
        if (a.kn) {
            const int n = a.kn[q.row_t];
            if (n >= 0) {
                if (chunk == 0) {
                    const double W = listed_resid_sum<BF16, NT>(a, q, n);
                    if (threadIdx.x < kSSub) out[threadIdx.x] = threadIdx.x == 0 ? W : 0.0;
                }
                return;
            }
        }
    }
    const uint8_t* trow = a.tgt + (size_t)q.row_t * a.V * Lt::ES;
    const uint8_t* drow = a.dft + (size_t)q.row_d * a.V * Lt::ES;
    chunk_weight_sums<BF16, VEC, NT>(trow, drow, a.V, chunk, q, q.c, true, a.topk != 0, red, out);
}

// One wave per request: beta_i = 1 - W_i (sums in a fixed order, clamped to [0, 1]), then
// E[A] = 1 + sum_j prod_{i<=j} beta_i. Failed requests get NaN (positions only when the
// offsets are sound).
template <bool BF16>
SD_DEV void accept_final_body(const SampleArgs& a, int b) {
    const int lane = threadIdx.x;
    const Decision r = a.rec[b];
    const bool cu_ok = !(r.mode == MODE_NONE && (r.flags & SPECDEC_ERR_K));
    const int lo = cu_ok ? a.cu[b] : 0;
    const int k = cu_ok ? a.cu[b + 1] - lo : 0;
    double beta = NAN;
    if (r.mode != MODE_NONE && lane < k) {
        const int pos = lo + lane;
        const double* w = a.wacc + (size_t)pos * a.nch * kSSub;
        bool listed = false;
        if constexpr (BF16) listed = a.kn && a.kn[a.prec[pos].row_t] >= 0;
        double W = 0.0;
        const int nsum = listed ? 1 : a.nch * kSSub;
        for (int i = 0; i < nsum; ++i) W += w[i];
        beta = fmin(1.0, fmax(0.0, 1.0 - W));
    }
    if (lane < k && a.dbg.accept_prob) a.dbg.accept_prob[lo + lane] = beta;
    double e = 1.0, run = 1.0;
    for (int i = 0; i < k; ++i) {
        run *= __shfl(beta, i, kWave);
        e += run;
    }
    if (lane == 0 && a.dbg.expected_emitted)
        a.dbg.expected_emitted[b] = r.mode == MODE_NONE ? (double)NAN : e;
}

// ---------------------------------------------------------------------------------------
// Per-request transform parameters. The row's request: for a target row r the b with
// cu[b] + b <= r < cu[b+1] + b + 1, for a draft row r' the b with cu[b] <= r' < cu[b+1]
// (a binary search over cu; a malformed cu is reported by the decision, the b found here
// only picks parameters). A request with invalid parameters gets c = 1 and no filter, so
// its rows are processed harmlessly, and the decision fails it with SPECDEC_ERR_PARAM.
// ---------------------------------------------------------------------------------------
struct ParamArgs {
    const int* cu;
    int B, K, V;
    const float* temp;       // [B] or null: the scalar T for every request
    const int* topk;         // [B] or null
    const float* topp;       // [B] or null
    float T;
    int top_k;
    float top_p;
    int top_k_max;           // requests with an active top_k above it fail
    int kc;                  // the chunk k of a top-p-alone row
    int tree;                // 1: draft rows laid out like target rows (trees: [K+B] each)
    RowParams* out;          // [2K+B], trees [2(K+B)]
};

SD_DEV RowParams row_params_of(const ParamArgs& a, int r) {
    const int rows_t = a.K + a.B;
    const bool tgt = r < rows_t;
    const int x = tgt ? r : r - rows_t;
    int lo = 0, hi = a.B;                       // largest b with start(b) <= x
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu[mid] + ((tgt || a.tree) ? mid : 0) <= x) lo = mid;
        else hi = mid;
    }
    const int b = lo;
    const float T = a.temp ? a.temp[b] : a.T;
    const int k = a.topk ? a.topk[b] : a.top_k;
    const float tp = a.topp ? a.topp[b] : a.top_p;
    const bool kon = k > 0 && k < a.V;
    const bool pon = tp > 0.0f && tp < 1.0f;
    const float c = (float)(1.4426950408889634074 / (double)T);   // log2(e) / T
    const bool bad = !(T > 0.0f) || !isfinite(T) || !(c > 0.0f) || !isfinite(c) || tp != tp ||
                     (kon && k > a.top_k_max);
    RowParams rp;
    if (bad) {
        rp.c = 1.0f;
        rp.k = 0;
        rp.top_p = 1.0f;
        rp.flags = kRpBad;
    } else {
        const int mode = kon ? 1 : (pon ? 2 : 0);
        rp.c = c;
        rp.k = mode == 1 ? k : (mode == 2 ? a.kc : 0);
        rp.top_p = pon ? tp : 1.0f;
        const bool generic = (mode == 1 && k > kTkMaxK) || (mode == 2 && a.kc >= a.V);
        rp.flags = mode | (generic ? kRpGeneric : 0);
    }
    return rp;
}

SD_DEV void row_params_one(const ParamArgs& a, int r) { a.out[r] = row_params_of(a, r); }

// One chunk of one row under per-request parameters: plain statistics into cpart for an
// unfiltered row, the candidate select otherwise (nothing for a row that takes the
// multi-pass select).
template <bool BF16, bool VEC>
SD_DEV void chunk_pr_body(const TopkArgs& a, int row, int chunk) {
    const RowParams rp = a.rpar[row];
    const int mode = rp.flags & kRpMode;
    const size_t ci = (size_t)row * a.nchunks + chunk;
    if (mode == 0) {
        row_stats_body<BF16, VEC>(a.tgt, a.dft, a.rows_t, a.V, a.nchunks, rp.c, a.cpart, (int)ci);
        if (threadIdx.x == 0) a.cnt[ci] = 0;
        return;
    }
    if (rp.flags & kRpGeneric) {
        if (threadIdx.x == 0) a.cnt[ci] = kTkWaves * a.wcap + 1;
        return;
    }
    topk_chunk_body<BF16, VEC, 2>(a, row, chunk, ChunkSel{rp.k, rp.c, mode == 2});
}

// The merge of one row under per-request parameters; an unfiltered row combines its chunk
// statistics (max, then the exp-sums rescaled to it in fp64, fixed order).
template <bool BF16, int NT>
SD_DEV void merge_pr_body(const TopkArgs& a, int row) {
    constexpr int LPT = kTkMaxChunks > NT ? kTkMaxChunks / NT : 1;
    const RowParams rp = a.rpar[row];
    const int mode = rp.flags & kRpMode;
    if (mode != 0) {
        topk_merge_body<BF16, NT>(a, row, RowSel{rp.k, mode == 2 ? 2 : (rp.top_p < 1.0f ? 1 : 0),
                                             rp.top_p, rp.c});
        return;
    }
    __shared__ float redf[NT / kWave];
    __shared__ double redd[NT / kWave];
    const int tid = threadIdx.x;
    const int nl = a.nchunks;
    RowPartial cp[LPT];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
        const int l = tid * LPT + q;
        cp[q] = l < nl ? a.cpart[(size_t)row * nl + l] : RowPartial{-INFINITY, 0, 0.0};
        mx = fmaxf(mx, cp[q].m);
    }
    const float m = block_max<NT>(mx, redf);
    double sp = 0.0;
#pragma unroll
    for (int q = 0; q < LPT; ++q)   // chunks with no finite entry carry 0 (or NaN)
        sp += cp[q].m == -INFINITY ? cp[q].s
                                   : cp[q].s * exp2(((double)cp[q].m - (double)m) * (double)rp.c);
    const double S = block_sum<NT>(sp, redd);
    if (tid == 0) {
        RowPartial out;
        out.m = m;
        out.nkept = -1;
        out.s = S;
        a.part[row] = out;
        a.row_thr[row] = -INFINITY;
        if (BF16 && a.kn && row < a.rows_t) a.kn[row] = -1;
    }
}

// ---------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Early exit with a top-k / top-p transform (scalar or per request). The position
// launches run the chunk select of the rows of live requests instead of their plain
// statistics (P2: 0 top-k, 1 top-p alone, 2 per-request parameters; the generic select of
// very large top_k has no chunk work), and a merge launch after each finishes those rows:
// the liveness test of the next launch reads the merged rows (one partial and a threshold
// per row), exactly what the decision reads.
template <bool BF16, bool VEC, int P2>
SD_DEV void chunk_of(const TopkArgs& ta, int row, int chunk) {
    if constexpr (P2 == 2) {
        chunk_pr_body<BF16, VEC>(ta, row, chunk);
    } else {
        if (ta.generic) return;
        topk_chunk_body<BF16, VEC, P2>(ta, row, chunk, ChunkSel{ta.top_k, ta.c, P2 == 1});
    }
}

template <bool BF16, bool VEC, int P2>
SD_DEV void fpass_body(const SampleArgs& a, const TopkArgs& ta, int p, int w) {
    pass_grid<BF16>(a, ta.nchunks, p, w,
                    [&](int row, int chunk) { chunk_of<BF16, VEC, P2>(ta, row, chunk); });
}

template <bool BF16, bool VEC, int P2>
SD_DEV void ftail_body(const SampleArgs& a, const TopkArgs& ta, int p, int w) {
    tail_grid<BF16, true>(a, ta.nchunks, p, w, true,
                    [&](int row, int chunk) { chunk_of<BF16, VEC, P2>(ta, row, chunk); });
}

// The merge of one row the launch before selected: at a position launch p < the tail's,
// workgroup w is (request w / 2, side w % 2) at p; after the tail launch at p, workgroup w
// is (request w / per, slot w % per) over the target rows p .. k_b (slots 0 .. k_b - p) and
// the draft rows p .. k_b - 1 (the slots after), per = 2 (max_k - p) + 1. Requests not
// live at p (the flag the launch before left) merge nothing.
template <bool BF16, int NT, bool PR>
SD_DEV void fmerge_body(const SampleArgs& a, const TopkArgs& ta, int p, int w, bool tail) {
    const int rows_t = a.K + a.B;
    const int per = tail ? early_tail_slots(a.max_k, p) : 2;
    const int b = w / per;
    const int j = w - b * per;
    const int lo = a.cu[b], hi = a.cu[b + 1];
    const int k = hi - lo;
    if (p > k || a.live[(p & 1) * a.B + b] == 0) return;
    int row;
    if (!tail) {
        if (j == 1 && p >= k) return;
        row = j == 0 ? lo + b + p : rows_t + lo + p;
    } else if (j <= k - p) {
        row = lo + b + p + j;                          // target rows p .. k
    } else {
        const int i = p + (j - (k - p + 1));           // draft rows p .. k - 1
        if (i >= k) return;
        row = rows_t + lo + i;
    }
    if constexpr (PR) merge_pr_body<BF16, NT>(ta, row);
    else topk_merge_body<BF16, NT>(ta, row, RowSel{ta.top_k, ta.topp_mode, ta.top_p, ta.c});
}

struct WsPlan {
    size_t part, thr, rec, wsum, live, tk_cnt, tk_cand, tk_kn, tk_ktok, tk_kkey, tk_cpart, tk_ctc,
        rpar, prec, wacc, total;
    int nparts, nchunks, nch, tk_wcap, tk_listed, filter, topp_mode, sel_k, sel_generic;
    int pr;                  // per-request parameters: every row through the chunk select
    int pr_plain;            // per-request temperatures only: plain statistics, per-row c
    int kc;                  // the chunk k of a top-p-alone row
};

// the transform arrays (stopping arrays alone keep the scalar path)
static inline bool per_request(const specdec_params* pr) {
    return pr && (pr->temperature || pr->top_k || pr->top_p);
}

static inline bool topk_active(int top_k, int V) { return top_k > 0 && top_k < V; }
static inline bool topp_active(float top_p) { return top_p > 0.0f && top_p < 1.0f; }
// 0: no top-p; 1: top-p inside the top-k set; 2: top-p alone
static inline int topp_mode(int top_k, float top_p, int V) {
    return !topp_active(top_p) ? 0 : (topk_active(top_k, V) ? 1 : 2);
}
// rows carry a threshold (top-k, top-p or both)
static inline bool filter_active(int top_k, float top_p, int V) {
    return topk_active(top_k, V) || topp_active(top_p);
}
// the k the chunk select runs with. Top-p alone asks each chunk for its top k_c tokens,
// k_c = kToppCand / nchunks (a multiple of 4 in [8, 128]); the per-thread-max bound then
// gathers about 1.5 kToppCand candidates per row on unstructured rows, within the merge's
// LDS, and the complete upper set above the largest chunk bound (about kToppCand tokens)
// is where the nucleus is searched.
static inline int select_k(int top_k, float top_p, int V, int nchunks) {
    if (topp_mode(top_k, top_p, V) != 2) return top_k;
    const int kc = (kToppCand / nchunks) & ~3;
    return kc < 8 ? 8 : (kc > 128 ? 128 : kc);
}
static inline bool select_generic(int top_k, float top_p, int V, int nchunks) {
    const int k = select_k(top_k, top_p, V, nchunks);
    return topk_generic(k) || k >= V;
}

// The transform's mode and the chunk select's k (no offsets yet).
static inline WsPlan plan_transform(int V, int dtype, int top_k, float top_p,
                                    const specdec_params* prm) {
    WsPlan p{};
    // the vector and scalar layouts use the same chunk length
    const int ch = dtype == SPECDEC_BF16 ? Layout<true, true>::CH : Layout<false, true>::CH;
    p.nchunks = (V + ch - 1) / ch;
    p.kc = select_k(0, 0.5f, V, p.nchunks);
    p.pr = per_request(prm);
    p.pr_plain = p.pr && !prm->top_k && !prm->top_p && !topk_active(top_k, V) &&
                 !topp_active(top_p);
    if (p.pr_plain) {
        // temperatures alone transform nothing but the exp-sums: the plain statistics, each
        // row with its request's log2(e) / T
        p.filter = 0;
        p.topp_mode = 0;
        p.sel_k = 0;
        p.sel_generic = 0;
    } else if (p.pr) {
        // lists sized for the largest chunk k any row may use
        int kmax = 0;
        if (prm->top_k) kmax = prm->top_k_max < kTkMaxK ? prm->top_k_max : kTkMaxK;
        else if (topk_active(top_k, V) && !topk_generic(top_k)) kmax = top_k;
        if (prm->top_p || topp_active(top_p)) kmax = kmax > p.kc ? kmax : p.kc;
        p.filter = 1;
        p.topp_mode = -1;               // per row
        p.sel_k = kmax > 0 ? kmax : 1;
        p.sel_generic = 0;
    } else {
        p.filter = filter_active(top_k, top_p, V);
        p.topp_mode = topp_mode(top_k, top_p, V);
        p.sel_k = select_k(top_k, top_p, V, p.nchunks);
        p.sel_generic = select_generic(top_k, top_p, V, p.nchunks);
    }
    p.nparts = p.filter ? 1 : p.nchunks;
    p.nch = (V + kSChunk - 1) / kSChunk;
    return p;
}

// The chunk select's lists from `off` for `rows` rows, the first rows_t of them target rows
// (listed: their kept tokens too, bf16 only); returns the end.
static inline size_t plan_select(WsPlan& p, size_t off, size_t rows, size_t rows_t, int dtype,
                                 bool listed) {
    p.tk_cnt = p.tk_cand = p.tk_cpart = p.tk_ctc = off;
    if (p.filter && !p.sel_generic) {
        p.tk_wcap = topk_wcap(p.sel_k);
        const size_t lists = rows * p.nchunks;
        off = align256(off + lists * sizeof(int));
        p.tk_cand = off;
        off = align256(off + lists * (size_t)topk_cstride(p.tk_wcap) * sizeof(uint32_t));
        if (p.topp_mode == 2 || p.pr) {    // per-chunk max / exp-sum and bound
            p.tk_cpart = off;
            off = align256(off + lists * sizeof(RowPartial));
            p.tk_ctc = off;
            off = align256(off + lists * sizeof(uint32_t));
        }
        if (listed && dtype == SPECDEC_BF16) {   // kept-token lists of the target rows
            p.tk_listed = 1;
            p.tk_kn = off;
            off = align256(off + rows_t * sizeof(int));
            p.tk_ktok = off;
            off = align256(off + rows_t * kKeptCap * sizeof(uint32_t));
            p.tk_kkey = off;
            off = align256(off + rows_t * kKeptCap * sizeof(uint16_t));
        }
    }
    return off;
}

static inline WsPlan plan_ws(int B, int K, int V, int dtype, int top_k, float top_p,
                             const specdec_params* prm) {
    WsPlan p = plan_transform(V, dtype, top_k, top_p, prm);
    const size_t rows = (size_t)2 * K + B;
    size_t off = 0;
    p.part = off;
    off = align256(off + rows * p.nparts * sizeof(RowPartial));
    p.thr = off;
    off = align256(off + rows * sizeof(float));
    p.rec = off;
    off = align256(off + (size_t)B * sizeof(Decision));
    p.wsum = off;
    off = align256(off + (size_t)B * p.nch * kSSub * sizeof(double));
    p.live = off;                          // early-exit liveness flags
    off = align256(off + (size_t)2 * B * sizeof(int));
    off = plan_select(p, off, rows, (size_t)K + B, dtype, true);
    p.rpar = off;
    if (p.pr) off = align256(off + rows * sizeof(RowParams));
    // acceptance analytics: a record and the sub-chunk residual sums of every position
    p.prec = off;
    off = align256(off + (size_t)K * sizeof(Decision));
    p.wacc = off;
    off = align256(off + (size_t)K * p.nch * kSSub * sizeof(double));
    p.total = off;
    return p;
}

static inline ParamArgs param_args(const int* cu, int B, int K, int V, float T, int top_k,
                                   float top_p, const specdec_params* prm, const WsPlan& p,
                                   uint8_t* ws) {
    ParamArgs a;
    a.cu = cu;
    a.B = B;
    a.K = K;
    a.V = V;
    a.temp = prm->temperature;
    a.topk = prm->top_k;
    a.topp = prm->top_p;
    a.T = T;
    a.top_k = top_k;
    a.top_p = top_p;
    a.top_k_max = prm->top_k ? prm->top_k_max : top_k;
    a.kc = p.kc;
    a.tree = 0;
    a.out = reinterpret_cast<RowParams*>(ws + p.rpar);
    return a;
}

static inline TopkArgs topk_args(const uint8_t* tgt, const uint8_t* dft, int rows_t, int V,
                                 float top_p, float c, const WsPlan& p, uint8_t* ws) {
    TopkArgs a;
    a.tgt = tgt;
    a.dft = dft;
    a.rows_t = rows_t;
    a.V = V;
    a.nchunks = p.nchunks;
    a.top_k = p.sel_k;
    a.wcap = p.tk_wcap;
    a.cstride = topk_cstride(p.tk_wcap);
    a.generic = p.sel_generic;
    a.c = c;
    a.cnt = reinterpret_cast<int*>(ws + p.tk_cnt);
    a.cand = reinterpret_cast<uint32_t*>(ws + p.tk_cand);
    a.kn = p.tk_listed ? reinterpret_cast<int*>(ws + p.tk_kn) : nullptr;
    a.ktok = p.tk_listed ? reinterpret_cast<uint32_t*>(ws + p.tk_ktok) : nullptr;
    a.kkey = p.tk_listed ? reinterpret_cast<uint16_t*>(ws + p.tk_kkey) : nullptr;
    a.part = reinterpret_cast<RowPartial*>(ws + p.part);
    a.row_thr = reinterpret_cast<float*>(ws + p.thr);
    a.topp_mode = p.topp_mode;
    a.top_p = top_p;
    const bool parts = p.topp_mode == 2 || p.pr;
    a.cpart = parts ? reinterpret_cast<RowPartial*>(ws + p.tk_cpart) : nullptr;
    a.ctc = parts ? reinterpret_cast<uint32_t*>(ws + p.tk_ctc) : nullptr;
    a.rpar = p.pr ? reinterpret_cast<const RowParams*>(ws + p.rpar) : nullptr;
    return a;
}

}  // namespace sd
