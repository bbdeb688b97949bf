// verify.hip -- batched lossless speculative-sampling verification and the
// analytic acceptance rate on gfx950.
//
// Method (pages cited by title and section):
//  * DART reading note (zhongzhuzhou.org), sec. 2.3, eq. (3)-(4): a draft token
//    x drawn from p is kept with probability min(1, q(x)/p(x)); otherwise the
//    token is redrawn from the residual [q - p]_+ / R, R = sum_v [q - p]_+, and
//    min(p, q) + R r = q makes the committed token's law exactly q.  At T = 0
//    verification compares with the target argmax.
//  * DSpark paper guide (personal-site-bgy.pages.dev), "speculative decoding
//    basics": strict left-to-right prefix survival, one bonus token from the
//    target when every draft passes; "confidence head": c* = 1 - 1/2 ||p - q||_1;
//    "scheduler": per-request verify length l_r.
//  * Speculative-decoding survey (zhifeiding.github.io), sec. 1.3: greedy
//    verification is a position-wise argmax comparison.
//
// Design (four launches per call, each a hand-off through the workspace):
//  * A "unit" is one position of one request: a (draft row, target row) pair
//    for positions i < l_r, the bonus target row at i = l_r.  Each unit's rows
//    are cut into C chunks of 64 N logits; one wave streams one chunk.
//  * Kernel 1 (stats_kernel, a persistent grid) reads every needed row
//    exactly once from HBM, chunk by chunk with the next chunk's 16-byte loads
//    in flight, and writes each chunk's max and exp-sum
//    sum 2^((z - m) s), s = log2(e) / T (or its argmax at T = 0).
//  * norm_kernel (one wave per unit) combines kernel 1's chunk statistics
//    into each row's normaliser (max M, Z = sum 2^((z - M) s)), or its argmax
//    at T = 0.
//  * Kernel 2 (tv_kernel, same structure as kernel 1) re-reads only the pair
//    rows -- kernel 1 has just streamed them, so they come from the 256 MB
//    Infinity Cache -- and reduces sum min(p, q) and sum [q - p]_+ per chunk.
//  * Kernel 3 (finalize_kernel, one workgroup per request): c* and Res (one
//    row per wave), the accept tests on the gathered
//    logits q(x), p(x) in fp64 (one position per lane, prefix survival by
//    ballot), and the residual or bonus draw as a two-level inverse CDF
//    (chunk masses, then one re-read chunk scanned in ascending token id).
#include <math.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <vector>


#include "common.h"

#ifndef SV_RING
#define SV_RING 2
#endif

namespace sv {

struct VerifyArgs {
    const void *zt;          // target logits
    const void *zd;          // draft logits
    const int32_t *tokens;   // [R][gamma]
    const int32_t *vlen;     // [R]
    const float *temp;       // [R]
    const float *ua;         // [R][gamma]
    const float *us;         // [R][gamma+1]
    int R, gamma, V;
    int C;                   // chunks per row
    int UG;                  // units per request (gamma + 1, or 1 for row pairs)
    int tG, dG;              // rows per request in the target / draft tensors
    int tv_mode;             // 1: independent row pairs, c* and Res only
    int32_t *out_tok;
    int32_t *out_n;
    float *out_cs;
    float *out_rs;
    float *out_lq;
    Control *ctl;
    float4 *st1;             // [units][C] chunk statistics (kernel 1)
    float2 *st2;             // [units][C] sum min / sum res of pair chunks (kernel 2)
    struct RowNorm *nrm;     // [units] row normalisers (norm_kernel)
};

// Normalisers of one unit's rows: at T > 0 the maxima and Z = sum 2^((z - M) s)
// of the target (t) and draft (d) rows; at T = 0 their argmax (-1: invalid).
struct RowNorm {
    float Mt, Md;
    int gt, gd;
    double Zt, Zd;
};

constexpr float kInf = __builtin_inff();

__device__ __forceinline__ bool temperature_ok(float T) {
    if (!(T >= 0.0f) || !(T <= 1e30f)) return false;  // NaN, negative, +inf, huge
    return T == 0.0f || T >= 1e-30f;
}
__device__ __forceinline__ bool uniform_ok(float u) { return u >= 0.0f && u < 1.0f; }

// exp2 scale of log2(e) / T, rounded to fp32 once; every workgroup of a
// request derives the same value.
__device__ __forceinline__ float exp2_scale(float T) { return (float)(kLog2e / (double)T); }

// Softmax arithmetic in scaled units.  With s = log2(e) / T a logit z has
// weight 2^(z s - mu) for any reference mu; the reference cancels in the
// normalisation, so every stage may pick its own as long as it scales
// consistently.  A chunk's reference is mu_c = fl(m_c s), its max logit times
// s rounded once, and an element's exponent is fma(z, s, -mu_c): a single
// rounding, tiny for the logits near the max that carry the mass.  Rounding
// is monotone, so the row's reference max_c mu_c is fl(M s).

// Exponent reference of a chunk with scaled max mu: mu itself, or 0 when the
// chunk holds no finite logit (then -inf gives weight 0, a NaN stays NaN).
__device__ __forceinline__ float exp_ref(float mu) { return (mu > -kInf) ? mu : 0.0f; }

// 2^(z s - ref) with the exponent from one fused multiply-add.
__device__ __forceinline__ float exp_w(float z, float s, float ref) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(z, s, -ref));
}

// Weight of a chunk with scaled max mu and exp-sum S relative to the row's
// scaled max muM: S * 2^(mu - muM), the power in fp32 (relative error ~1e-7,
// like the fp32 exp-sums), accumulated by callers in fp64.  Shared by every
// stage that combines a row, so all obtain identical normalisers.
__device__ __forceinline__ double chunk_weight(float mu, float S, float muM) {
    return (mu > -kInf) ? (double)S * (double)__builtin_amdgcn_exp2f(mu - muM) : 0.0;
}

// Probability scale of a chunk: p_v = 2^(z_v s - mu) * scale.
__device__ __forceinline__ float chunk_scale(float mu, float muM, double Z) {
    return (mu > -kInf) ? (float)((double)__builtin_amdgcn_exp2f(mu - muM) / Z) : 0.0f;
}

// [q - p]_+ computed as q - min(p, q) with rounded products (no contraction),
// identical wherever it is evaluated.
__device__ __forceinline__ void pq_weights(float et, float ed, float at, float ad, float &q,
                                           float &mn) {
    q = __fmul_rn(et, at);
    float p = __fmul_rn(ed, ad);
    mn = fminf(p, q);
}


__device__ void write_invalid(const VerifyArgs &a, int r) {
    const float nan = __builtin_nanf("");
    if (a.tv_mode) {
        a.out_cs[r] = nan;
        if (a.out_rs) a.out_rs[r] = nan;
    } else {
        for (int j = 0; j <= a.gamma; ++j) {
            a.out_tok[(size_t)r * (a.gamma + 1) + j] = -1;
            if (a.out_lq) a.out_lq[(size_t)r * (a.gamma + 1) + j] = nan;
        }
        for (int i = 0; i < a.gamma; ++i) {
            if (a.out_cs) a.out_cs[(size_t)r * a.gamma + i] = nan;
            if (a.out_rs) a.out_rs[(size_t)r * a.gamma + i] = nan;
        }
        a.out_n[r] = -1;
    }
    atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
}

// ---------------------------------------------------------------------------
// chunk items: one wave streams one chunk of kLanes * N logits per row
// ---------------------------------------------------------------------------

constexpr int kLanes = 64;

struct Item {
    int u, r, i, c, l;
    float T, s;   // temperature and log2(e) / T
    bool pair;    // the draft row is present (i < l)
};

// Global wave index and wave count of the launch (each wave works alone).
__device__ __forceinline__ long wave_index() {
    return (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
}
__device__ __forceinline__ long wave_count() { return (long)gridDim.x * kWaves; }

// Walks this wave's items wave_index() + k * wave_count() in increasing k and
// yields the active ones.  The wave decides the activity of 64 candidates at
// once (lane k holds candidate base + k and its request parameters) and hands
// them out in order with readlane, so the item loop issues no loads of its
// own; one round of loads per 64 candidates.
struct ItemCursor {
    long base = -64;
    uint64_t mask = 0;
    int lr = 0, li = 0, lc = 0, ll = 0;
    float lT = 0.0f, ls = 0.0f;

    // pairs_only: yield only pair items at T > 0 (the ones kernel 2 reduces)
    __device__ bool next(const VerifyArgs &a, long work, Item &x, bool pairs_only = false) {
        const long W = wave_count(), w0 = wave_index();
        for (;;) {
            if (mask) {
                const int k = __builtin_ctzll(mask);
                mask &= mask - 1;
                x.r = __builtin_amdgcn_readlane(lr, k);
                x.i = __builtin_amdgcn_readlane(li, k);
                x.c = __builtin_amdgcn_readlane(lc, k);
                x.l = __builtin_amdgcn_readlane(ll, k);
                x.T = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lT), k));
                x.s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), k));
                x.u = x.r * a.UG + x.i;
                x.pair = x.i < x.l;
                return true;
            }
            base += 64;
            if (w0 + base * W >= work) return false;
            const long it = w0 + (base + (threadIdx.x & 63)) * W;
            bool act = false;
            if (it < work) {
                const int u = (int)(it / a.C);
                lc = (int)(it % a.C);
                lr = u / a.UG;
                li = u % a.UG;
                lT = a.temp[lr];
                ll = a.tv_mode ? 1 : a.vlen[lr];
                act = temperature_ok(lT) && ll >= 0 && ll <= a.gamma && li <= ll;
                if (pairs_only) act = act && li < ll && lT != 0.0f;
                ls = act && lT != 0.0f ? exp2_scale(lT) : 0.0f;
            }
            mask = __ballot(act);
        }
    }
};

// Raw register image of one row chunk, N logits per lane.  With vector loads
// (EPV > 1) bf16 logits stay packed two per word; on the scalar path every
// logit is widened to fp32 when loaded.
template <typename T, int N, int EPV>
struct RawChunk {
    static constexpr bool kPacked = (EPV > 1) && (EltBytes<T>::value == 2);
    static constexpr int kWords = kPacked ? N / 2 : N;
    uint32_t w[kWords];

    // Slot j * EPV + q of lane l holds logit c0 + (j * 64 + l) * EPV + q, so
    // each load instruction of the wave reads consecutive 16-byte pieces.
    // A chunk inside the row (all but the last) loads without bounds checks;
    // past the row end a vector holds -inf (V % EPV == 0 when EPV > 1).
    __device__ __forceinline__ void load(const T *row, long c0, int V) {
        const int lane = threadIdx.x & 63;
        if (c0 + (long)kLanes * N <= V) {
#pragma unroll
            for (int j = 0; j < N / EPV; ++j)
                load_vec(row, c0 + ((long)j * kLanes + lane) * EPV, j, true);
        } else {
#pragma unroll
            for (int j = 0; j < N / EPV; ++j) {
                const long e = c0 + ((long)j * kLanes + lane) * EPV;
                load_vec(row, e, j, e < V);
            }
        }
    }

    __device__ __forceinline__ void load_vec(const T *row, long e, int j, bool in) {
        if constexpr (EPV == 1) {
            w[j] = __float_as_uint(in ? load_one(row, e) : -kInf);
        } else if constexpr (kPacked) {
            constexpr int NW = EPV / 2;
            if constexpr (NW == 4) {
                uint4 v = in ? *reinterpret_cast<const uint4 *>(row + e)
                             : make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
                w[j * 4 + 0] = v.x; w[j * 4 + 1] = v.y; w[j * 4 + 2] = v.z; w[j * 4 + 3] = v.w;
            } else if constexpr (NW == 2) {
                uint2 v = in ? *reinterpret_cast<const uint2 *>(row + e)
                             : make_uint2(0xff80ff80u, 0xff80ff80u);
                w[j * 2 + 0] = v.x; w[j * 2 + 1] = v.y;
            } else {
                w[j] = in ? *reinterpret_cast<const uint32_t *>(row + e) : 0xff80ff80u;
            }
        } else {
            if constexpr (EPV == 4) {
                uint4 v = in ? *reinterpret_cast<const uint4 *>(row + e)
                             : make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
                w[j * 4 + 0] = v.x; w[j * 4 + 1] = v.y; w[j * 4 + 2] = v.z; w[j * 4 + 3] = v.w;
            } else {
                uint2 v = in ? *reinterpret_cast<const uint2 *>(row + e)
                             : make_uint2(0xff800000u, 0xff800000u);
                w[j * 2 + 0] = v.x; w[j * 2 + 1] = v.y;
            }
        }
    }

    __device__ __forceinline__ float get(int k) const {
        if constexpr (kPacked) return (k & 1) ? bf16_hi(w[k >> 1]) : bf16_lo(w[k >> 1]);
        else return __uint_as_float(w[k]);
    }
};

template <int N>
__device__ __forceinline__ long chunk_start(int c) { return (long)c * kLanes * N; }

template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ void load_item(const VerifyArgs &a, const Item &x,
                                          RawChunk<TT, N, EPV> &rt, RawChunk<TD, N, EPV> &rd) {
    const long c0 = chunk_start<N>(x.c);
    rt.load((const TT *)a.zt + ((long)x.r * a.tG + x.i) * a.V, c0, a.V);
    if (x.pair) rd.load((const TD *)a.zd + ((long)x.r * a.dG + x.i) * a.V, c0, a.V);
}

// ---------------------------------------------------------------------------
// kernel 1: per-chunk statistics (every needed row, read once from HBM)
// ---------------------------------------------------------------------------

// Chunk c of unit u (one wave): scaled max mu = fl(m s) and exp-sum
// S = sum 2^(z s - mu) of the target row (and of the draft row for pairs)
// -> st1[u * C + c] = (mu_t, S_t, mu_d, S_d); at T = 0 the argmax (value,
// index; index 0xffffffff if a NaN was seen).
template <bool PAIR, typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ void chunk_stats_t(const VerifyArgs &a, const Item &x,
                                              const RawChunk<TT, N, EPV> &rt,
                                              const RawChunk<TD, N, EPV> &rd) {
    const int lane = threadIdx.x & 63;
    float4 *out = a.st1 + (size_t)x.u * a.C + x.c;
    if (x.T == 0.0f) {
        const long c0 = chunk_start<N>(x.c);
        float bt = -kInf, bd = -kInf;
        int it = 0x7fffffff, id = 0x7fffffff, bad = 0;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int e = (int)(c0 + ((long)(k / EPV) * kLanes + lane) * EPV + (k % EPV));
            const float zt = rt.get(k);
            if (zt != zt) bad |= 1;
            if (zt > bt) { bt = zt; it = e; }
            if constexpr (PAIR) {
                const float zd = rd.get(k);
                if (zd != zd) bad |= 2;
                if (zd > bd) { bd = zd; id = e; }
            }
        }
        wave_argmax(bt, it);
        if constexpr (PAIR) wave_argmax(bd, id);
        bad = wave_max_i(bad);
        if (lane == 0)
            *out = make_float4(bt, __uint_as_float((bad & 1) ? 0xffffffffu : (uint32_t)it), bd,
                               __uint_as_float((bad & 2) ? 0xffffffffu : (uint32_t)id));
        return;
    }
    const float s = x.s;
    float mt = -kInf, md = -kInf;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        mt = fmaxf(mt, rt.get(k));
        if constexpr (PAIR) md = fmaxf(md, rd.get(k));
    }
    const float mut = wave_max(mt) * s;
    const float mud = PAIR ? wave_max(md) * s : -kInf;
    const float rt0 = exp_ref(mut), rd0 = exp_ref(mud);
    float et = 0.0f, ed = 0.0f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        et += exp_w(rt.get(k), s, rt0);
        if constexpr (PAIR) ed += exp_w(rd.get(k), s, rd0);
    }
    const float st = wave_sum_f(et);
    const float sd = PAIR ? wave_sum_f(ed) : 0.0f;
    if (lane == 0) *out = make_float4(mut, st, mud, sd);
}

template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ void chunk_stats(const VerifyArgs &a, const Item &x,
                                            const RawChunk<TT, N, EPV> &rt,
                                            const RawChunk<TD, N, EPV> &rd) {
    if (x.pair) chunk_stats_t<true>(a, x, rt, rd);
    else chunk_stats_t<false>(a, x, rt, rd);
}

// Persistent loop of one wave over its items with a ring of kRing register
// buffers: while the wave reduces item k, the loads of items k+1 .. k+kRing-1
// are in flight.  Op::apply(a, item, target chunk, draft chunk) is the
// per-item work.
constexpr int kRing = SV_RING;

template <typename Op, typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ void run_items(const VerifyArgs &a, bool pairs_only) {
    const long work = (long)a.R * a.UG * a.C;
    ItemCursor cur;
    Item x[kRing];
    bool has[kRing];
    RawChunk<TT, N, EPV> t[kRing];
    RawChunk<TD, N, EPV> d[kRing];
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) {
        has[k] = cur.next(a, work, x[k], pairs_only);
        if (has[k]) load_item(a, x[k], t[k], d[k]);
    }
    has[kRing - 1] = false;
    for (;;) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
            const int pf = (k + kRing - 1) % kRing;
            has[pf] = has[(pf + kRing - 1) % kRing] && cur.next(a, work, x[pf], pairs_only);
            __asm__ volatile("" ::: "memory");
            if (has[pf]) load_item(a, x[pf], t[pf], d[pf]);
            if (!has[k]) return;
            Op::apply(a, x[k], t[k], d[k]);
        }
    }
}

struct StatsOp {
    template <typename TT, typename TD, int N, int EPV>
    __device__ __forceinline__ static void apply(const VerifyArgs &a, const Item &x,
                                                 const RawChunk<TT, N, EPV> &rt,
                                                 const RawChunk<TD, N, EPV> &rd) {
        chunk_stats<TT, TD, N, EPV>(a, x, rt, rd);
    }
};

// Kernel 1, a persistent grid of independent waves.
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kBlock) stats_kernel(VerifyArgs a) {
    run_items<StatsOp, TT, TD, N, EPV>(a, false);
}

// ---------------------------------------------------------------------------
// kernel 2: sum min(p, q) and sum [q - p]_+ per chunk, then the finalisers
// ---------------------------------------------------------------------------

struct FinalState {
    float Mt[kMaxGamma + 1], Md[kMaxGamma];
    double Zt[kMaxGamma + 1], Zd[kMaxGamma];
    double cs[kMaxGamma], rs[kMaxGamma];
    int gt[kMaxGamma + 1], gd[kMaxGamma];
    int rowok[kMaxGamma + 1];
    float lq[kMaxGamma + 1];
    int A, ok, csel, resid, token;
    double tsel;
    float ztok;
};

// Row normalisers of unit u from kernel 1's chunk statistics, by one wave
// (lanes over chunks): the scaled maxima muM and Z = sum_c S_c 2^(mu_c - muM).
__device__ void wave_row_stats(const VerifyArgs &a, int u, bool pair, float &Mt, double &Zt,
                               float &Md, double &Zd) {
    const int lane = threadIdx.x & 63;
    const float4 *st = a.st1 + (size_t)u * a.C;
    float mt = -kInf, md = -kInf;
    for (int c = lane; c < a.C; c += 64) {
        const float4 v = st[c];
        mt = fmaxf(mt, v.x);
        if (pair) md = fmaxf(md, v.z);
    }
    Mt = wave_max(mt);
    Md = wave_max(md);
    double zt = 0.0, zd = 0.0;
    for (int c = lane; c < a.C; c += 64) {
        const float4 v = st[c];
        zt += chunk_weight(v.x, v.y, Mt);
        if (pair) zd += chunk_weight(v.z, v.w, Md);
    }
    Zt = wave_sum(zt);
    Zd = wave_sum(zd);
}

// Argmax of a row (and of its draft row) from kernel 1's words (T = 0), by one
// wave; -1 for an invalid row.
__device__ void wave_row_argmax(const VerifyArgs &a, int u, bool pair, int &gt, int &gd) {
    const int lane = threadIdx.x & 63;
    const float4 *st = a.st1 + (size_t)u * a.C;
    float vt = -kInf, vd = -kInf;
    int it = 0x7fffffff, id = 0x7fffffff, bad = 0;
    for (int c = lane; c < a.C; c += 64) {
        const float4 v = st[c];
        const uint32_t ti = __float_as_uint(v.y), di = __float_as_uint(v.w);
        if (ti == 0xffffffffu) bad = 1;
        else argmax_combine(vt, it, v.x, (int)ti);
        if (pair) {
            if (di == 0xffffffffu) bad = 1;
            else argmax_combine(vd, id, v.z, (int)di);
        }
    }
    wave_argmax(vt, it);
    wave_argmax(vd, id);
    bad = wave_max_i(bad);
    gt = (!bad && vt < kInf && it != 0x7fffffff) ? it : -1;
    gd = pair ? ((!bad && vd < kInf && id != 0x7fffffff) ? id : -1) : 0;
}

// Inverse-CDF draw inside chunk c of row j of request r by the workgroup (cmt,
// cmd: the chunk's exponent references, at, ad: its probability scales): the
// first logit (ascending id) whose running weight exceeds tsel, with weights
// q - min(p, q) (resid) or q, computed exactly as kernel 2 computed them.
// Thread t owns logits [c0 + t P, c0 + (t+1) P), P = 64 N / 256; a block scan
// finds the owner, which walks its logits again.  Clamps to the chunk's last
// positive weight.
template <typename TT, typename TD, int N, int EPV>
__device__ int draw_in_chunk(const VerifyArgs &a, int r, int j, int c, bool resid, float s,
                             float cmt, float cmd, float at, float ad, double tsel, float *ztok,
                             BlockScratch &bs, FinalState &f) {
    constexpr int PER = kLanes * N / kBlock;          // logits per thread
    constexpr int VW = (EPV < PER) ? EPV : PER;       // vector width of its loads
    const int tid = threadIdx.x;
    const int V = a.V;
    const long c0 = chunk_start<N>(c);
    const long e0 = c0 + (long)tid * PER;
    const TT *trow = (const TT *)a.zt + ((long)r * a.tG + j) * V;
    const TD *drow = resid ? (const TD *)a.zd + ((long)r * a.dG + j) * V : nullptr;
    auto weights = [&](long e, float *w, float *zo) {
        float zt[VW], zd[VW];
        if (e < V) {
            VecLoad<TT, VW>::run(trow, e, zt);
            if (resid) VecLoad<TD, VW>::run(drow, e, zd);
        } else {
#pragma unroll
            for (int q = 0; q < VW; ++q) zt[q] = zd[q] = -kInf;
        }
#pragma unroll
        for (int q = 0; q < VW; ++q) {
            const float et = exp_w(zt[q], s, cmt);
            if (resid) {
                const float ed = exp_w(zd[q], s, cmd);
                float qv, mn;
                pq_weights(et, ed, at, ad, qv, mn);
                w[q] = qv - mn;
            } else {
                w[q] = __fmul_rn(et, at);
            }
            zo[q] = zt[q];
        }
    };
    double tot = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int k = 0; k < PER; k += VW) {
        float w[VW], z[VW];
        weights(e0 + k, w, z);
#pragma unroll
        for (int q = 0; q < VW; ++q) {
            tot += (double)w[q];
            if (w[q] > 0.0f) lastpos = k + q;
        }
    }
    double all;
    const double excl = block_exclusive_scan(tot, &all, bs);
    const int owner = block_min_i((tot > 0.0 && excl + tot > tsel) ? tid : 0x7fffffff, bs);
    if (owner == 0x7fffffff) {
        // tsel at or past the chunk's total (rounding): last positive weight;
        // if every fp32 weight underflowed, the chunk's first logit
        const int last = block_max_i(lastpos >= 0 ? (int)(e0 + lastpos) : -1, bs);
        const int tok = last >= 0 ? last : (int)c0;
        *ztok = load_one(trow, tok);
        return tok;
    }
    if (tid == owner) {
        double cum = excl;
        int tok = -1;
        float zz = 0.0f;
        for (int k = 0; k < PER && tok < 0; k += VW) {
            float w[VW], z[VW];
            weights(e0 + k, w, z);
#pragma unroll
            for (int q = 0; q < VW; ++q) {
                cum += (double)w[q];
                if (tok < 0 && cum > tsel) {
                    tok = (int)(e0 + k + q);
                    zz = z[q];
                }
            }
        }
        if (tok < 0) {  // tot > 0, so lastpos >= 0
            tok = (int)(e0 + lastpos);
            zz = load_one(trow, tok);
        }
        f.token = tok;
        f.ztok = zz;
    }
    __syncthreads();
    *ztok = f.ztok;
    return f.token;
}

// Final outputs of request r: accept tests, prefix survival, the residual or
// bonus draw and the commit (or c* / Res for independent row pairs).  Every
// input it reads was written by kernels 1 and 2 before this launch.
template <typename TT, typename TD, int N, int EPV>
__device__ void finalize(const VerifyArgs &a, const Item &x, BlockScratch &bs, FinalState &f) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int G = a.gamma, V = a.V, C = a.C, r = x.r, l = x.l;
    const float T = x.T;
    const float nan = __builtin_nanf("");
    const int nrows = a.tv_mode ? 1 : l + 1;
    const int npairs = a.tv_mode ? 1 : l;
    const int u0 = r * a.UG;
    if (tid == 0) f.ok = 1;
    __syncthreads();

    if (T == 0.0f) {
        for (int i = wave; i < nrows; i += kWaves) {
            const RowNorm nm = a.nrm[u0 + i];
            const int gt = nm.gt, gd = nm.gd;
            if (lane == 0) {
                f.gt[i] = gt;
                if (i < l) f.gd[i] = gd;
                if (gt < 0 || (i < l && gd < 0)) f.ok = 0;
            }
        }
        __syncthreads();
        if (wave != 0) return;
        if (!f.ok) { if (lane == 0) write_invalid(a, r); return; }
        if (a.tv_mode) {
            if (lane == 0) {
                const float cv = (f.gt[0] == f.gd[0]) ? 1.0f : 0.0f;
                a.out_cs[r] = cv;
                if (a.out_rs) a.out_rs[r] = 1.0f - cv;
            }
            return;
        }
        bool bad = false, acc = false;
        if (lane < l) {
            const int xv = a.tokens[(size_t)r * G + lane];
            bad = xv < 0 || xv >= V;
            acc = !bad && xv == f.gt[lane];
        }
        const uint64_t badm = __ballot(bad), accm = __ballot(acc);
        if (badm) { if (lane == 0) write_invalid(a, r); return; }
        int A = (~accm == 0) ? 64 : __builtin_ctzll(~accm);
        if (A > l) A = l;
        const int gA = f.gt[A];
        int32_t *tok = a.out_tok + (size_t)r * (G + 1);
        for (int k = lane; k <= G; k += 64) {
            tok[k] = (k < A) ? a.tokens[(size_t)r * G + k] : (k == A ? gA : -1);
            if (a.out_lq) a.out_lq[(size_t)r * (G + 1) + k] = (k <= A) ? 0.0f : nan;
        }
        for (int i = lane; i < G; i += 64) {
            const float cv = (i < l) ? ((f.gt[i] == f.gd[i]) ? 1.0f : 0.0f) : nan;
            if (a.out_cs) a.out_cs[(size_t)r * G + i] = cv;
            if (a.out_rs) a.out_rs[(size_t)r * G + i] = (i < l) ? 1.0f - cv : nan;
        }
        if (lane == 0) a.out_n[r] = A;
        return;
    }

    // ---- T > 0: row normalisers and c* / Res, one row per wave -------------
    const float s = exp2_scale(T);
    for (int i = wave; i < nrows; i += kWaves) {
        const bool pair = i < l;
        const RowNorm nm = a.nrm[u0 + i];
        const float Mt = nm.Mt, Md = nm.Md;
        const double Zt = nm.Zt, Zd = nm.Zd;
        double dm = 0.0, dr = 0.0;
        if (pair) {
            for (int c = lane; c < C; c += 64) {
                const float2 w = a.st2[(size_t)(u0 + i) * C + c];
                dm += (double)w.x;
                dr += (double)w.y;
            }
            dm = wave_sum(dm);
            dr = wave_sum(dr);
        }
        if (lane == 0) {
            f.Mt[i] = Mt;
            f.Zt[i] = Zt;
            bool ok = (Mt > -kInf) && (Mt < kInf) && (Zt > 0.0) && (Zt < 1e300);
            if (pair) {
                f.Md[i] = Md;
                f.Zd[i] = Zd;
                f.cs[i] = dm;
                f.rs[i] = dr;
                ok = ok && (Md > -kInf) && (Md < kInf) && (Zd > 0.0) && (Zd < 1e300);
            }
            if (!ok) f.ok = 0;
        }
    }
    __syncthreads();
    if (a.tv_mode) {
        if (tid == 0) {
            if (!f.ok) { write_invalid(a, r); return; }
            a.out_cs[r] = (float)f.cs[0];
            if (a.out_rs) a.out_rs[r] = (float)f.rs[0];
        }
        return;
    }

    // ---- accept tests (lane i tests position i), prefix survival by ballot --
    if (wave == 0) {
        bool bad = !f.ok, acc = false;
        for (int j2 = lane; j2 <= l; j2 += 64)
            bad = bad || !uniform_ok(a.us[(size_t)r * (G + 1) + j2]);
        if (lane < l) {
            const int xv = a.tokens[(size_t)r * G + lane];
            const float u = a.ua[(size_t)r * G + lane];
            bad = bad || xv < 0 || xv >= V || !uniform_ok(u);
            if (!bad) {
                const TT *trow = (const TT *)a.zt + ((long)r * a.tG + lane) * V;
                const TD *drow = (const TD *)a.zd + ((long)r * a.dG + lane) * V;
                const double lq = (double)load_one(trow, xv) * (double)s - (double)f.Mt[lane];
                const double lp = (double)load_one(drow, xv) * (double)s - (double)f.Md[lane];
                const double q = exp2(lq) / f.Zt[lane];
                const double p = exp2(lp) / f.Zd[lane];
                acc = q >= p || (double)u < q / p;
                f.lq[lane] = (float)(lq * kLn2 - log(f.Zt[lane]));
            }
        }
        const uint64_t badm = __ballot(bad), accm = __ballot(acc);
        if (lane == 0) {
            const int A = (~accm == 0) ? 64 : __builtin_ctzll(~accm);
            f.A = A > l ? l : A;
            f.ok = badm == 0;
        }
    }
    __syncthreads();
    if (!f.ok) {
        if (tid == 0) write_invalid(a, r);
        return;
    }
    const int A = f.A, j = A;
    const int uj = u0 + j;
    const float Mt = f.Mt[j];
    const double Zt = f.Zt[j];

    // ---- chunk masses of the final draw and the chunk holding u * W --------
    if (wave == 0) {
        bool resid = A < l;
        double W = 0.0;
        if (resid) {
            for (int c = lane; c < C; c += 64) W += (double)a.st2[(size_t)uj * C + c].y;
            W = wave_sum(W);
            if (!(W > 0.0)) resid = false;  // no residual mass (rounding): draw from q
        }
        if (!resid) {
            W = 0.0;
            for (int c = lane; c < C; c += 64) {
                const float4 v = a.st1[(size_t)uj * C + c];
                W += chunk_weight(v.x, v.y, Mt) / Zt;
            }
            W = wave_sum(W);
        }
        const double t = (double)a.us[(size_t)r * (G + 1) + j] * W;
        int csel = -1, clast = -1;
        double tsel = 0.0, run = 0.0;
        for (int cb = 0; cb < C && csel < 0; cb += 64) {
            const int c = cb + lane;
            double wc = 0.0;
            if (c < C) {
                if (resid) {
                    wc = (double)a.st2[(size_t)uj * C + c].y;
                } else {
                    const float4 v = a.st1[(size_t)uj * C + c];
                    wc = chunk_weight(v.x, v.y, Mt) / Zt;
                }
            }
            double incl = wc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const double nb = __shfl_up(incl, o, 64);
                if (lane >= o) incl += nb;
            }
            const double excl = run + incl - wc;
            const uint64_t hit = __ballot(c < C && excl + wc > t);
            const uint64_t pos = __ballot(c < C && wc > 0.0);
            if (pos) clast = cb + 63 - __builtin_clzll(pos);
            if (hit) {
                csel = cb + __builtin_ctzll(hit);
                tsel = __shfl(t - excl, csel - cb, 64);
            }
            run += __shfl(incl, 63, 64);
        }
        if (csel < 0) {  // t at or past the total (rounding): last chunk with mass
            csel = clast >= 0 ? clast : 0;
            tsel = INFINITY;
        }
        if (lane == 0) {
            f.csel = csel;
            f.tsel = tsel;
            f.resid = resid;
        }
    }
    __syncthreads();
    const int csel = f.csel;
    const bool resid = f.resid;
    const float4 cst = a.st1[(size_t)uj * C + csel];
    const float cmt = exp_ref(cst.x);
    const float cmd = resid ? exp_ref(cst.z) : 0.0f;
    const float at = chunk_scale(cst.x, Mt, Zt);
    const float ad = resid ? chunk_scale(cst.z, f.Md[j], f.Zd[j]) : 0.0f;
    float ztok;
    const int token = draw_in_chunk<TT, TD, N, EPV>(a, r, j, csel, resid, s, cmt, cmd, at, ad,
                                                    f.tsel, &ztok, bs, f);
    if (wave == 0) {
        const float lqj = (float)(((double)ztok * (double)s - (double)Mt) * kLn2 - log(Zt));
        int32_t *tok = a.out_tok + (size_t)r * (G + 1);
        for (int k = lane; k <= G; k += 64) {
            tok[k] = (k < A) ? a.tokens[(size_t)r * G + k] : (k == A ? token : -1);
            if (a.out_lq)
                a.out_lq[(size_t)r * (G + 1) + k] = (k < A) ? f.lq[k] : (k == A ? lqj : nan);
        }
        for (int i = lane; i < G; i += 64) {
            if (a.out_cs) a.out_cs[(size_t)r * G + i] = (i < l) ? (float)f.cs[i] : nan;
            if (a.out_rs) a.out_rs[(size_t)r * G + i] = (i < l) ? (float)f.rs[i] : nan;
        }
        if (lane == 0) a.out_n[r] = A;
    }
}

// Kernel 2 work for one pair item at T > 0 (one wave): sum min(p, q) and
// sum [q - p]_+ over the chunk, with the row normalisers of norm_kernel
// -> st2[u * C + c].
template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ void chunk_tv(const VerifyArgs &a, const Item &x,
                                         const RawChunk<TT, N, EPV> &rt,
                                         const RawChunk<TD, N, EPV> &rd) {
    const int lane = threadIdx.x & 63;
    const float s = x.s;
    const RowNorm nm = a.nrm[x.u];
    const float4 own = a.st1[(size_t)x.u * a.C + x.c];
    const float at = chunk_scale(own.x, nm.Mt, nm.Zt);
    const float ad = chunk_scale(own.z, nm.Md, nm.Zd);
    const float rt0 = exp_ref(own.x), rd0 = exp_ref(own.z);
    float smin = 0.0f, sres = 0.0f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float et = exp_w(rt.get(k), s, rt0);
        const float ed = exp_w(rd.get(k), s, rd0);
        float q, mn;
        pq_weights(et, ed, at, ad, q, mn);
        smin += mn;
        sres += q - mn;
    }
    const float dm = wave_sum_f(smin);
    const float dr = wave_sum_f(sres);
    if (lane == 0) a.st2[(size_t)x.u * a.C + x.c] = make_float2(dm, dr);
}

struct TvOp {
    template <typename TT, typename TD, int N, int EPV>
    __device__ __forceinline__ static void apply(const VerifyArgs &a, const Item &x,
                                                 const RawChunk<TT, N, EPV> &rt,
                                                 const RawChunk<TD, N, EPV> &rd) {
        chunk_tv<TT, TD, N, EPV>(a, x, rt, rd);
    }
};

// Kernel 2, a persistent grid of independent waves over the pair items at
// T > 0 with the same load ring as kernel 1.  The rows it re-reads were
// streamed by kernel 1 moments before, so they come from the 256 MB Infinity
// Cache.
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kBlock) tv_kernel(VerifyArgs a) {
    run_items<TvOp, TT, TD, N, EPV>(a, true);
}

// Row normalisers (T > 0) or argmaxes (T = 0) of every active unit, one wave
// per unit, from kernel 1's chunk statistics.
__global__ void __launch_bounds__(kBlock) norm_kernel(VerifyArgs a) {
    const long u = wave_index();
    if (u >= (long)a.R * a.UG) return;
    const int r = (int)(u / a.UG), i = (int)(u % a.UG);
    const float T = a.temp[r];
    const int l = a.tv_mode ? 1 : a.vlen[r];
    if (!(temperature_ok(T) && l >= 0 && l <= a.gamma && i <= l)) return;
    const bool pair = i < l;
    RowNorm nm;
    if (T == 0.0f) {
        wave_row_argmax(a, (int)u, pair, nm.gt, nm.gd);
        nm.Mt = nm.Md = 0.0f;
        nm.Zt = nm.Zd = 0.0;
    } else {
        wave_row_stats(a, (int)u, pair, nm.Mt, nm.Zt, nm.Md, nm.Zd);
        nm.gt = nm.gd = 0;
    }
    if ((threadIdx.x & 63) == 0) a.nrm[u] = nm;
}

// Kernel 3: one workgroup per request writes its final outputs (or the
// invalid-request outputs).
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kBlock) finalize_kernel(VerifyArgs a) {
    __shared__ BlockScratch bs;
    __shared__ FinalState f;
    Item x;
    x.r = blockIdx.x;
    x.T = a.temp[x.r];
    x.l = a.tv_mode ? 1 : a.vlen[x.r];
    if (!(temperature_ok(x.T) && x.l >= 0 && x.l <= a.gamma)) {
        if (threadIdx.x == 0) write_invalid(a, x.r);
        return;
    }
    finalize<TT, TD, N, EPV>(a, x, bs, f);
}

__global__ void zero_fill_kernel(uint32_t *p, size_t n_words) {
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n_words;
         k += (size_t)gridDim.x * blockDim.x)
        p[k] = 0u;
}

__global__ void clear_status_kernel(Control *ctl) { atomic_store_u32(&ctl->status, 0u); }

// ---------------------------------------------------------------------------
// host side: plan, validation, dispatch
// ---------------------------------------------------------------------------

namespace {

constexpr long kTargetItems = 65536;   // chunk items wanted: several per resident wave

struct Plan {
    int N;           // logits per thread per row
    int C;           // chunks per row
    long units;
    size_t off_st1, off_st2, off_nrm, bytes;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int forced_n() {
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("SPECVERIFY_CHUNK_N");
        v = e ? atoi(e) : 0;
        if (v != 4 && v != 8 && v != 16 && v != 32) v = 0;
    }
    return v;
}

// Largest per-thread chunk that still gives enough workgroups; the smallest
// one otherwise.  Returns false if V needs more than kMaxChunks chunks.
bool make_plan(long R, long units_per_req, long V, Plan &p) {
    static const int kN[] = {32, 16, 8, 4};
    const long units = R * units_per_req;
    int chosen = -1, chosen_C = 0;
    for (int N : kN) {
        const long C = (V + (long)kLanes * N - 1) / ((long)kLanes * N);
        if (C > kMaxChunks) continue;
        chosen = N;
        chosen_C = (int)C;
        if (forced_n() == N) break;
        if (!forced_n() && units * C >= kTargetItems) break;
    }
    if (chosen < 0) return false;
    if (units * (long)chosen_C > 0x7fffffffL) return false;
    p.N = chosen;
    p.C = chosen_C;
    p.units = units;
    p.off_st1 = sizeof(Control);
    p.off_st2 = round_up(p.off_st1 + sizeof(float4) * (size_t)units * chosen_C, 256);
    p.off_nrm = round_up(p.off_st2 + sizeof(float2) * (size_t)units * chosen_C, 256);
    p.bytes = round_up(p.off_nrm + sizeof(RowNorm) * (size_t)units, 256);
    return true;
}

bool dtype_ok(int d) { return d == SPEC_F32 || d == SPEC_BF16; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Workgroups of a persistent grid: the kernel's resident capacity on the
// current device (cached per kernel and device), at most `items`.
long grid_for(const void *kernel, long items) {
    struct Entry { const void *k; int dev; long cap; };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return items;
    long cap = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : cache)
            if (e.k == kernel && e.dev == dev) cap = e.cap;
        if (cap == 0) {
            int nb = 0, ncu = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kBlock, 0) != hipSuccess ||
                hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
                return items;
            cap = (long)(nb > 0 ? nb : 1) * (ncu > 0 ? ncu : 1);
            cache.push_back(Entry{kernel, dev, cap});
        }
    }
    return items < cap ? items : cap;
}

template <typename TT, typename TD, int N, int EPV>
int launch_kernels(const VerifyArgs &a, long items, hipStream_t st) {
    const void *k1 = reinterpret_cast<const void *>(&stats_kernel<TT, TD, N, EPV>);
    const void *k2 = reinterpret_cast<const void *>(&tv_kernel<TT, TD, N, EPV>);
    const long wgs = (items + kWaves - 1) / kWaves;  // one item per wave at a time
    long g1 = grid_for(k1, wgs), g2 = grid_for(k2, wgs);
    if (g1 < 1) g1 = 1;
    if (g2 < 1) g2 = 1;
    static bool said = false;
    if (!said && getenv("SPECVERIFY_VERBOSE")) {
        said = true;
        fprintf(stderr, "[specverify] verify N=%d EPV=%d C=%d items=%ld grids %ld / %ld\n", N,
                EPV, a.C, items, g1, g2);
    }
    hipLaunchKernelGGL((stats_kernel<TT, TD, N, EPV>), dim3((unsigned)g1), dim3(kBlock), 0, st, a);
    const long units = (long)a.R * a.UG;
    hipLaunchKernelGGL(norm_kernel, dim3((unsigned)((units + kWaves - 1) / kWaves)), dim3(kBlock),
                       0, st, a);
    hipLaunchKernelGGL((tv_kernel<TT, TD, N, EPV>), dim3((unsigned)g2), dim3(kBlock), 0, st, a);
    hipLaunchKernelGGL((finalize_kernel<TT, TD, N, EPV>), dim3((unsigned)a.R), dim3(kBlock), 0, st,
                       a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

template <typename TT, typename TD, int N>
int launch_n(const VerifyArgs &a, bool vec, long items, hipStream_t st) {
    constexpr int eb = (EltBytes<TT>::value > EltBytes<TD>::value) ? EltBytes<TT>::value
                                                                   : EltBytes<TD>::value;
    constexpr int ev = (16 / eb < N) ? 16 / eb : N;
    return vec ? launch_kernels<TT, TD, N, ev>(a, items, st)
               : launch_kernels<TT, TD, N, 1>(a, items, st);
}

template <typename TT, typename TD>
int launch_types(const VerifyArgs &a, int N, bool vec, long items, hipStream_t st) {
    switch (N) {
        case 32: return launch_n<TT, TD, 32>(a, vec, items, st);
        case 16: return launch_n<TT, TD, 16>(a, vec, items, st);
        case 8: return launch_n<TT, TD, 8>(a, vec, items, st);
        case 4: return launch_n<TT, TD, 4>(a, vec, items, st);
    }
    return SPEC_EUNSUPPORTED;
}

int launch(const VerifyArgs &a, int tdt, int ddt, int N, bool vec, long items, hipStream_t st) {
    if (tdt == SPEC_BF16 && ddt == SPEC_BF16)
        return launch_types<uint16_t, uint16_t>(a, N, vec, items, st);
    if (tdt == SPEC_F32 && ddt == SPEC_F32) return launch_types<float, float>(a, N, vec, items, st);
    if (tdt == SPEC_BF16 && ddt == SPEC_F32)
        return launch_types<uint16_t, float>(a, N, vec, items, st);
    return launch_types<float, uint16_t>(a, N, vec, items, st);
}

void bind_workspace(VerifyArgs &a, void *ws, const Plan &p) {
    char *b = (char *)ws;
    a.ctl = (Control *)b;
    a.st1 = (float4 *)(b + p.off_st1);
    a.st2 = (float2 *)(b + p.off_st2);
    a.nrm = (RowNorm *)(b + p.off_nrm);
    a.C = p.C;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

int spec_version(void) { return 100; }

const char *spec_status_string(int status) {
    switch (status) {
        case SPEC_OK: return "SPEC_OK";
        case SPEC_EINVAL: return "SPEC_EINVAL: null required pointer or invalid size";
        case SPEC_EDTYPE: return "SPEC_EDTYPE: unsupported dtype";
        case SPEC_EWORKSPACE: return "SPEC_EWORKSPACE: workspace null, too small or misaligned";
        case SPEC_EHIP: return "SPEC_EHIP: HIP runtime call or kernel launch failed";
        case SPEC_EUNSUPPORTED: return "SPEC_EUNSUPPORTED: shape outside the supported range";
    }
    return "unknown spec_status";
}

size_t spec_verify_workspace_bytes(int R, int gamma, int V) {
    if (R < 0 || gamma < 0 || gamma > kMaxGamma || V < 1 || V > SPEC_MAX_VOCAB) return 0;
    Plan p;
    if (!make_plan(R > 0 ? R : 1, gamma + 1, V, p)) return 0;
    return p.bytes;
}

size_t spec_tv_workspace_bytes(int N, int V) {
    if (N < 0 || V < 1 || V > SPEC_MAX_VOCAB) return 0;
    Plan p;
    if (!make_plan(N > 0 ? N : 1, 1, V, p)) return 0;
    return p.bytes;
}

int spec_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace || workspace_bytes < sizeof(Control) || ((uintptr_t)workspace & 255u))
        return SPEC_EWORKSPACE;
    const size_t words = workspace_bytes / 4;
    const size_t blocks = (words + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                       dim3(kBlock), 0, (hipStream_t)stream, (uint32_t *)workspace, words);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int spec_get_device_status(void *workspace, uint32_t *host_bits, int clear, void *stream) {
    if (!workspace || !host_bits) return SPEC_EINVAL;
    Control *ctl = (Control *)workspace;
    hipStream_t st = (hipStream_t)stream;
    if (hipStreamSynchronize(st) != hipSuccess) return SPEC_EHIP;
    if (hipMemcpy(host_bits, &ctl->status, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return SPEC_EHIP;
    if (clear) {
        hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, st, ctl);
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
        if (hipStreamSynchronize(st) != hipSuccess) return SPEC_EHIP;
    }
    return SPEC_OK;
}

int spec_verify_batch(const void *target_logits, int t_dtype, const void *draft_logits,
                      int d_dtype, const int32_t *draft_tokens, const int32_t *verify_len,
                      const float *temperature, const float *u_accept, const float *u_sample,
                      int R, int gamma, int V, int32_t *out_tokens, int32_t *out_num_accepted,
                      float *out_cstar, float *out_resid_mass, float *out_logq, void *workspace,
                      size_t workspace_bytes, void *stream) {
    if (R < 0 || gamma < 0 || V < 1) return SPEC_EINVAL;
    if (!dtype_ok(t_dtype) || !dtype_ok(d_dtype)) return SPEC_EDTYPE;
    if (gamma > kMaxGamma || V > SPEC_MAX_VOCAB) return SPEC_EUNSUPPORTED;
    if (R == 0) return SPEC_OK;
    if (!target_logits || !verify_len || !temperature || !u_sample || !out_tokens ||
        !out_num_accepted)
        return SPEC_EINVAL;
    if (gamma > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SPEC_EINVAL;
    Plan p;
    if (!make_plan(R, gamma + 1, V, p)) return SPEC_EUNSUPPORTED;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < p.bytes)
        return SPEC_EWORKSPACE;
    VerifyArgs a{};
    a.zt = target_logits;
    a.zd = draft_logits;
    a.tokens = draft_tokens;
    a.vlen = verify_len;
    a.temp = temperature;
    a.ua = u_accept;
    a.us = u_sample;
    a.R = R;
    a.gamma = gamma;
    a.V = V;
    a.UG = gamma + 1;
    a.tG = gamma + 1;
    a.dG = gamma;
    a.tv_mode = 0;
    a.out_tok = out_tokens;
    a.out_n = out_num_accepted;
    a.out_cs = out_cstar;
    a.out_rs = out_resid_mass;
    a.out_lq = out_logq;
    bind_workspace(a, workspace, p);
    const bool vec = (V % 8 == 0) && aligned16(target_logits) &&
                     (gamma == 0 || aligned16(draft_logits));
    return launch(a, t_dtype, d_dtype, p.N, vec, p.units * p.C, (hipStream_t)stream);
}

int spec_tv_accept_rate(const void *draft_logits, const void *target_logits, int dtype,
                        const float *temperature, int N, int V, float *out_cstar,
                        float *out_resid_mass, void *workspace, size_t workspace_bytes,
                        void *stream) {
    if (N < 0 || V < 1) return SPEC_EINVAL;
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (V > SPEC_MAX_VOCAB) return SPEC_EUNSUPPORTED;
    if (N == 0) return SPEC_OK;
    if (!draft_logits || !target_logits || !temperature || !out_cstar) return SPEC_EINVAL;
    Plan p;
    if (!make_plan(N, 1, V, p)) return SPEC_EUNSUPPORTED;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < p.bytes)
        return SPEC_EWORKSPACE;
    VerifyArgs a{};
    a.zt = target_logits;
    a.zd = draft_logits;
    a.temp = temperature;
    a.R = N;
    a.gamma = 1;
    a.V = V;
    a.UG = 1;
    a.tG = 1;
    a.dG = 1;
    a.tv_mode = 1;
    a.out_cs = out_cstar;
    a.out_rs = out_resid_mass;
    bind_workspace(a, workspace, p);
    const bool vec = (V % 8 == 0) && aligned16(target_logits) && aligned16(draft_logits);
    return launch(a, dtype, dtype, p.N, vec, p.units * p.C, (hipStream_t)stream);
}

}  // extern "C"
