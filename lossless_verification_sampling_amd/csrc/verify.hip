// verify.hip -- batched lossless speculative-sampling verification and the
// analytic acceptance rate on gfx950: stream-ordered launches, two or four
// per call.
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
// Design.  A "unit" is one position of one request: the (target, draft) row
// pair of position i < l_r, or the bonus target row i = l_r.  Each unit's rows
// are cut into C chunks of 64 N logits, and an "item" is one chunk of one
// unit.  The split path (any dtypes and sizes) takes four launches, in
// stream order:
//  1. stats_kernel: persistent wave64s stream every needed row exactly once
//     from HBM with 16-byte loads, the items balanced over the waves through a
//     per-block unit table in LDS.  Per item it writes the chunk's scaled max
//     mu and weight sum S = sum 2^(z s - mu) per row (s = log2(e) / T), or the
//     chunk argmax at T = 0.
//  2. fold_kernel: one wave per draft position at T > 0 folds the chunk words
//     into the row normalisers (M = max mu, Z = sum S 2^(mu - M)) and every
//     chunk's pair scale (the factors that put the two rows' chunk weights on
//     one probability scale), and runs the accept test on the two gathered
//     logits of the draft token.
//  3. tv_kernel: the pair items at T > 0 again -- launch 1 has just streamed
//     them, so they come from the 256 MB Infinity Cache when they fit -- with
//     each chunk's weights rebuilt exactly as launch 1 made them; per item
//     the chunk's sum min(p, q) and residual mass sum [q - p]_+.
//  4. combine_kernel: one workgroup per request.  Its waves summarise the
//     request's units (accept flags, c*, Res, the chunk each row would draw
//     from); prefix survival then fixes the number of accepted drafts, and
//     the workgroup makes the one draw the request commits (the residual at
//     the first rejection, or the bonus from q; at T = 0 the target argmax)
//     and writes the outputs.  Row-pair mode (c* and Res only) takes one wave
//     per pair instead.
// The held path replaces launches 1-3 for bf16 rows of more than 64 chunks
// (at most two pairs per compute unit): hold_kernel gives each row pair at
// T > 0 one workgroup, which keeps 64 of its chunks in registers and as many
// more as shared memory holds (38 at R = 64, gamma = 7, V = 151936) from the
// statistics pass to the TV pass, folds
// the normalisers and pair scales in every wave and reads only the rest of
// the pair again; the workgroups without a pair stream the other rows (bonus
// rows, T = 0 rows) for their statistics.  It writes the same words, bit for
// bit, and the combine follows unchanged.
// No launch waits on a word of its own launch: each reads only what earlier
// launches of the call wrote.  Those words are 64-bit (launch tag, payload)
// pairs, so a reader never mistakes a stale word (an earlier call's, say
// after a launch failed) for a current one.  The tag is kept on the device,
// so that a captured graph gets a new one at every replay: launch 1 reads the
// workspace's next tag and copies it to the call's slot, the later launches
// read that slot, and the combine (the last launch) stores the tag after it
// as the next.  A word
// that is still stale when read raises SPEC_DEV_SPIN_TIMEOUT after a bounded
// re-poll instead of being used.
#include <math.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "common.h"

namespace sv {

constexpr float kInf = __builtin_inff();
constexpr int kLanes = 64;
// waves per SIMD the streaming kernels are compiled for (their registers fit)
constexpr int kStreamWaves = 5;

// Per-unit record words (tagged), filled by the unit's combines and read by
// the request's finaliser.
enum : int { kRecFlags = 0, kRecLqx = 1, kRecDraw = 2, kRecLqd = 3, kRecCs = 4, kRecRs = 5,
             kRecWords = 8 };
constexpr uint32_t kFlagValid = 1u, kFlagAccept = 2u;

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
    uint32_t tag;            // the call's tag (nonzero, top bit set), read on the device
    int compact;             // streaming kernels walk a unit table in LDS (else all candidates)
    int32_t *out_tok;
    int32_t *out_n;
    float *out_cs;
    float *out_rs;
    float *out_lq;
    Control *ctl;
    uint64_t *st1;           // [units][C][4] chunk stats
    uint64_t *st2;           // [units][C][2] chunk sum min(p, q), residual mass
    uint64_t *nrm;           // [units][4] unit normalisers
    uint64_t *rec;           // [units][kRecWords] unit records
    uint64_t *psc;           // [units * C][4] per-chunk pair scales (chi, clo, unit)
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ bool temperature_ok(float T) {
    if (!(T >= 0.0f) || !(T <= 1e30f)) return false;  // NaN, negative, +inf, huge
    return T == 0.0f || T >= 1e-30f;
}
__device__ __forceinline__ bool uniform_ok(float u) { return u >= 0.0f && u < 1.0f; }
__device__ __forceinline__ bool finite_f(float x) { return x - x == 0.0f; }

// exp2 scale log2(e) / T rounded to fp32 once; every wave derives the same value.
__device__ __forceinline__ float exp2_scale(float T) { return (float)(kLog2e / (double)T); }

// Exponent reference of a chunk with scaled max mu: mu itself, or 0 when the
// chunk holds no finite logit (-inf then gives weight 0, a NaN stays NaN).
__device__ __forceinline__ float exp_ref(float mu) { return (mu > -kInf) ? mu : 0.0f; }

// 2^(z s - ref), the exponent from one fused multiply-add: a single rounding,
// tiny for the logits near the chunk max that carry the mass.
__device__ __forceinline__ float ew(float z, float s, float ref) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(z, s, -ref));
}

// Probability scale of a chunk (p_v = e_v * alpha) from its scaled max mu and
// the row normalisers (M = max over chunks of mu, Z = sum 2^(z s - M)).
__device__ __forceinline__ float chunk_alpha(float mu, float M, float Z) {
    return (mu > -kInf) ? (float)((double)__builtin_amdgcn_exp2f(mu - M) / (double)Z) : 0.0f;
}

// Agent-scope 64-bit words: (tag << 32) | payload.
__device__ __forceinline__ uint64_t ld_word(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t *p, uint32_t tag, uint32_t payload) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Words w0..w(n-1) at p[0..n-1] (n <= 4) with no branch: every lane stores,
// lanes n.. the last word again (the same value to the same address), so
// that the compiler's count of memory operations in flight stays exact for
// the waits on loads issued before it.
__device__ __forceinline__ void publish_all(uint64_t *p, uint32_t tag, int n, uint32_t w0,
                                            uint32_t w1, uint32_t w2, uint32_t w3) {
    const int k = min(lane_id(), n - 1);
    const uint32_t w = k == 0 ? w0 : k == 1 ? w1 : k == 2 ? w2 : w3;
    st_word(p + k, tag, w);
}

// Lanes 0..n-1 store words w[lane] at p[lane] (n <= 4).
__device__ __forceinline__ void publish_n(uint64_t *p, uint32_t tag, int n, uint32_t w0,
                                          uint32_t w1, uint32_t w2, uint32_t w3) {
    const int lane = lane_id();
    if (lane < n) {
        const uint32_t w = lane == 0 ? w0 : lane == 1 ? w1 : lane == 2 ? w2 : w3;
        st_word(p + lane, tag, w);
    }
}

// The call's tag: launch 1 takes the workspace's next tag (0 after
// initialisation) and records it for the later launches.  Both slots are
// written by one thread of one workgroup and read with plain loads in later
// launches (a kernel boundary orders them): stores from every workgroup to
// one address would hold up each wave's first loads.
__device__ __forceinline__ uint32_t first_launch_tag(Control *ctl) {
    const uint32_t t = __builtin_amdgcn_readfirstlane(ctl->tag_next) | 0x80000000u;
    if (blockIdx.x == 0 && threadIdx.x == 0) ctl->tag_call = t;
    return t;
}
__device__ __forceinline__ uint32_t call_tag(const Control *ctl) {
    return __builtin_amdgcn_readfirstlane(ctl->tag_call);
}

__device__ __forceinline__ uint32_t rl(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ float rlf(float v, int l) { return readlane_f(v, l); }

// ---------------------------------------------------------------------------
// items
// ---------------------------------------------------------------------------

struct Item {
    int u, r, i, c, l;
    float T, s;   // temperature and log2(e) / T (0 at T = 0)
};
__device__ __forceinline__ bool is_pair(const Item &x) { return x.i < x.l; }

// The wave's index in the grid, made explicitly wave-uniform (the compiler
// cannot tell that threadIdx.x / 64 is the same in every lane of a wave), so
// that everything derived from it stays in scalar registers and branches.
__device__ __forceinline__ long wave_index() {
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    return (long)blockIdx.x * kWaves + w;
}
__device__ __forceinline__ long wave_count() { return (long)gridDim.x * kWaves; }

// Request r's (T, l) and whether the request is well formed.
__device__ __forceinline__ bool request_ok(const VerifyArgs &a, int r, float &T, int &l) {
    T = a.temp[r];
    l = a.tv_mode ? 1 : a.vlen[r];
    return temperature_ok(T) && l >= 0 && l <= a.gamma;
}

// Walks this wave's items wave_index() + k * wave_count() in increasing k and
// yields the active ones (units i <= l_r of well-formed requests).  Lane j
// judges candidate base + j, so one round of loads serves 64 candidates.
struct ItemCursor {
    uint32_t base = 0;       // candidate round: candidates w0 + (base + j) W
    uint64_t mask = 0;
    int lr = 0, li = 0, lc = 0, ll = 0;
    float lT = 0.0f, ls = 0.0f;
    bool first = true;

    // work < 2^31 (checked by the host), so 32-bit indices suffice.
    // tv_only: yield only pair items at T > 0 (the TV pass's items).
    __device__ bool next(const VerifyArgs &a, uint32_t work, Item &x, bool tv_only) {
        const uint32_t W = (uint32_t)wave_count(), w0 = (uint32_t)wave_index();
        for (;;) {
            if (mask) {
                const int k = __builtin_ctzll(mask);
                mask &= mask - 1;
                x.r = __builtin_amdgcn_readlane(lr, k);
                x.i = __builtin_amdgcn_readlane(li, k);
                x.c = __builtin_amdgcn_readlane(lc, k);
                x.l = __builtin_amdgcn_readlane(ll, k);
                x.T = rlf(lT, k);
                x.s = rlf(ls, k);
                x.u = x.r * a.UG + x.i;
                return true;
            }
            if (!first) base += 64;
            first = false;
            // first candidate of this round; rounds past the end stop
            if ((uint64_t)w0 + (uint64_t)base * W >= work) return false;
            const uint64_t it64 = (uint64_t)w0 + (uint64_t)(base + (uint32_t)lane_id()) * W;
            bool act = false;
            if (it64 < work) {
                const uint32_t it = (uint32_t)it64;
                const uint32_t u = it / (uint32_t)a.C;
                lc = (int)(it - u * (uint32_t)a.C);
                lr = (int)(u / (uint32_t)a.UG);
                li = (int)(u - (uint32_t)lr * (uint32_t)a.UG);
                act = request_ok(a, lr, lT, ll) && li <= ll;
                if (tv_only) act = act && li < ll && lT != 0.0f;
                ls = (act && lT != 0.0f) ? exp2_scale(lT) : 0.0f;
            }
            mask = __ballot(act);
        }
    }
};

// Work list of the streaming kernels when the unit table fits in LDS: every
// workgroup lists the active units (request-major) in shared memory at launch,
// and item k (unit k / C, chunk k % C) belongs to wave k mod W.  Only active
// items are enumerated, so every wave gets the same number of items (+-1).
// Shared layout: req[3 R] = (T, s, l) per request, then units[] = r << 7 | i.
struct UnitTable {
    const uint32_t *req;
    const uint32_t *units;
    uint32_t items;  // active units * C
};

// Units of one request in the table: positions 0..l (the TV pass: the pairs
// 0..l-1 at T > 0), never more than the request's UG unit slots (row pairs
// have no bonus unit).
__device__ __forceinline__ int table_units(const VerifyArgs &a, bool ok, float T, int l,
                                           bool tv_only) {
    if (!ok) return 0;
    const int n = tv_only ? (T != 0.0f ? l : 0) : l + 1;
    return n < a.UG ? n : a.UG;
}

// Builds the table in shared memory `lds` (all threads of the block).  tv_only
// lists the pair units at T > 0 only.
__device__ __forceinline__ UnitTable build_unit_table(const VerifyArgs &a, uint32_t *lds,
                                                      bool tv_only) {
    __shared__ uint32_t wsum[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t *req = lds;
    uint32_t *units = lds + 3 * a.R;
    // thread t owns requests [t K, t K + K)
    const int K = (a.R + kBlock - 1) / kBlock;
    const int r0 = tid * K, r1 = min(r0 + K, a.R);
    uint32_t own = 0;
    for (int r = r0; r < r1; ++r) {
        float T;
        int l;
        const bool ok = request_ok(a, r, T, l);
        req[3 * r + 0] = __float_as_uint(T);
        req[3 * r + 1] = __float_as_uint(ok && T != 0.0f ? exp2_scale(T) : 0.0f);
        req[3 * r + 2] = (uint32_t)l;
        own += (uint32_t)table_units(a, ok, T, l, tv_only);
    }
    // block exclusive scan of the per-thread unit counts
    const uint32_t incl = wave_incl_scan_dpp(own);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) base += wsum[w];
        total += wsum[w];
    }
    uint32_t pos = base + incl - own;
    for (int r = r0; r < r1; ++r) {
        const int l = (int)req[3 * r + 2];
        const float T = __uint_as_float(req[3 * r]);
        const bool ok = temperature_ok(T) && l >= 0 && l <= a.gamma;
        const int n = table_units(a, ok, T, l, tv_only);
        for (int i = 0; i < n; ++i) units[pos++] = ((uint32_t)r << 7) | (uint32_t)i;
    }
    __syncthreads();
    UnitTable t;
    t.req = req;
    t.units = units;
    t.items = total * (uint32_t)a.C;
    return t;
}

struct CompactCursor {
    uint32_t k;
    __device__ bool next(const VerifyArgs &a, const UnitTable &t, Item &x) {
        if (k >= t.items) return false;
        const uint32_t U = k / (uint32_t)a.C;
        x.c = (int)(k - U * (uint32_t)a.C);
        k += (uint32_t)wave_count();
        const uint32_t e = __builtin_amdgcn_readfirstlane(t.units[U]);
        x.r = (int)(e >> 7);
        x.i = (int)(e & 127u);
        x.T = __uint_as_float(__builtin_amdgcn_readfirstlane(t.req[3 * x.r]));
        x.s = __uint_as_float(__builtin_amdgcn_readfirstlane(t.req[3 * x.r + 1]));
        x.l = (int)__builtin_amdgcn_readfirstlane(t.req[3 * x.r + 2]);
        x.u = x.r * a.UG + x.i;
        return true;
    }
};

// Either cursor behind one interface.
struct Walker {
    bool compact;
    UnitTable t;
    CompactCursor cc;
    ItemCursor ic;
    uint32_t work;
    bool tv_only;
    __device__ bool next(const VerifyArgs &a, Item &x) {
        return compact ? cc.next(a, t, x) : ic.next(a, work, x, tv_only);
    }
};

__device__ __forceinline__ Walker make_walker(const VerifyArgs &a, uint32_t *lds, bool tv_only) {
    Walker w;
    w.compact = a.compact != 0;
    w.tv_only = tv_only;
    w.work = (uint32_t)a.R * (uint32_t)a.UG * (uint32_t)a.C;
    w.cc.k = (uint32_t)wave_index();
    if (w.compact) w.t = build_unit_table(a, lds, tv_only);
    return w;
}

// ---------------------------------------------------------------------------
// chunk registers
// ---------------------------------------------------------------------------

// Raw register image of one row chunk, N logits per lane.  Slot j * EPV + q of
// lane l holds logit c0 + (j * 64 + l) * EPV + q, so each load instruction of
// the wave reads consecutive 16-byte pieces.  bf16 logits stay packed two per
// word with vector loads; the scalar path (EPV == 1) widens them at load time.
template <typename T, int N, int EPV>
struct RawChunk {
    static constexpr bool kPacked = (EPV > 1) && (EltBytes<T>::value == 2);
    static constexpr int kWords = kPacked ? N / 2 : N;
    uint32_t w[kWords];

    int rem;  // ids of the chunk inside the row (64 N except in the last chunk)

    // Issues the chunk's loads unconditionally, in one basic block, so that
    // the compiler can wait for exactly these loads later: a vector past the
    // row end re-reads the chunk's first vector (inside the row) and is turned
    // into -inf by fix() (V % EPV == 0 when EPV > 1).
    __device__ __forceinline__ void load(const T *row, long c0, int V) {
        const T *base = row + c0;
        const uint32_t lane = (uint32_t)lane_id();
        const long left = (long)V - c0;
        rem = left < (long)kLanes * N ? (int)left : kLanes * N;
#pragma unroll
        for (int j = 0; j < N / EPV; ++j) {
            const uint32_t e = (j * kLanes + lane) * EPV;
            load_vec(base, (int)e < rem ? e : 0u, j);
        }
    }

    // Marks the vectors past the row end -inf; call before using the words.
    __device__ __forceinline__ void fix() {
        if (rem == kLanes * N) return;
        const uint32_t lane = (uint32_t)lane_id();
#pragma unroll
        for (int j = 0; j < N / EPV; ++j) {
            const bool out = (int)((j * kLanes + lane) * EPV) >= rem;
            constexpr int WPV = kWords / (N / EPV);  // words per vector
#pragma unroll
            for (int q = 0; q < WPV; ++q)
                if (out) w[j * WPV + q] = kPacked ? 0xff80ff80u : 0xff800000u;
        }
    }

    __device__ __forceinline__ void load_vec(const T *base, uint32_t e, int j) {
        if constexpr (EPV == 1) {
            w[j] = __float_as_uint(load_one(base, (long)e));
        } else if constexpr (kPacked) {
            constexpr int NW = EPV / 2;
            if constexpr (NW == 4) {
                const uint4 v = *reinterpret_cast<const uint4 *>(base + e);
                w[j * 4 + 0] = v.x; w[j * 4 + 1] = v.y; w[j * 4 + 2] = v.z; w[j * 4 + 3] = v.w;
            } else {
                static_assert(NW == 2, "bf16 vector width");
                const uint2 v = *reinterpret_cast<const uint2 *>(base + e);
                w[j * 2 + 0] = v.x; w[j * 2 + 1] = v.y;
            }
        } else {
            static_assert(EPV == 4, "fp32 vector width");
            const uint4 v = *reinterpret_cast<const uint4 *>(base + e);
            w[j * 4 + 0] = v.x; w[j * 4 + 1] = v.y; w[j * 4 + 2] = v.z; w[j * 4 + 3] = v.w;
        }
    }

    __device__ __forceinline__ float get(int k) const {
        if constexpr (kPacked) return (k & 1) ? bf16_hi(w[k >> 1]) : bf16_lo(w[k >> 1]);
        else return __uint_as_float(w[k]);
    }
};

// Token id of slot k of this lane in the chunk starting at c0.
template <int EPV>
__device__ __forceinline__ int slot_id(long c0, int k) {
    return (int)(c0 + ((long)(k / EPV) * kLanes + lane_id()) * EPV + (k % EPV));
}

template <typename TT, typename TD, int N>
struct ChunkGeom {
    static constexpr int kEB = (EltBytes<TT>::value > EltBytes<TD>::value) ? EltBytes<TT>::value
                                                                          : EltBytes<TD>::value;
    static constexpr int kVec = (16 / kEB < N) ? 16 / kEB : N;
};

template <typename T>
__device__ __forceinline__ const T *row_ptr(const void *base, int r, int G, int i, int V) {
    return (const T *)base + ((long)r * G + i) * V;
}

// ---------------------------------------------------------------------------
// per-chunk reductions
// ---------------------------------------------------------------------------

// Sum of the N values of a lane in slot order.  Every sum over a chunk's
// weights goes through this function, so sums of identical weights are
// bitwise identical wherever they are taken.
template <int N>
__device__ __forceinline__ float lane_sum(const float (&v)[N]) {
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < N; ++k) acc += v[k];
    return acc;
}

// T > 0: scaled chunk max mu = fl(m s), weights e_k = 2^(z_k s - mu) (kept in
// e) and their wave sum S.
template <int N, typename RC>
__device__ __forceinline__ void chunk_exp(const RC &raw, float s, float (&e)[N], float &mu,
                                          float &S) {
    float m = -kInf;
#pragma unroll
    for (int k = 0; k < N; ++k) m = __builtin_elementwise_maximum(m, raw.get(k));
    mu = wave_max(m) * s;
    const float ref = exp_ref(mu);
#pragma unroll
    for (int k = 0; k < N; ++k) e[k] = ew(raw.get(k), s, ref);
    S = wave_sum_f(lane_sum<N>(e));
}

// T = 0: chunk argmax (value, index; lowest index on ties); bad = a NaN seen.
template <int N, int EPV, typename RC>
__device__ __forceinline__ void chunk_argmax(const RC &raw, long c0, float &bv, int &bi,
                                             int &bad) {
    bv = -kInf;
    bi = 0x7fffffff;
    bad = 0;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float z = raw.get(k);
        if (z != z) bad = 1;
        if (z > bv) {
            bv = z;
            bi = slot_id<EPV>(c0, k);
        }
    }
    wave_argmax(bv, bi);
    bad = wave_max_i(bad);
}

// Scaling of a row pair's chunk weights for min(p, q).  With q_v = e_t alpha_t
// and p_v = e_d alpha_d (e = 2^(z s - ref), alpha = 2^(mu - M) / Z per row),
// min(p, q) in units of alpha_t is 2^min(a, b): a = z_t s - ref_t is the
// target weight's exponent and b = z_d s + c the draft weight's on the
// target's scale, c = -ref_d + log2(alpha_d / alpha_t).  One exponential per
// element, and where the target side is the smaller the term is the target
// weight bit for bit, so a chunk where q <= p everywhere leaves a residual of
// exactly 0.  c is carried as a float pair (chi + clo); both scales are at
// least 2^-149 / V when nonzero, so |log2(alpha_d / alpha_t)| < 170.
struct PairScale {
    float unit;       // alpha_t; 0 where q vanishes on the chunk (its terms are 0)
    float chi, clo;   // c = chi + clo
};

// A row's normalisers with the reciprocal of Z taken once (fp64).
struct RowNorm {
    float M, Z;
    double rZ;
};
__device__ __forceinline__ RowNorm row_norm(float M, float Z) {
    RowNorm n;
    n.M = M;
    n.Z = Z;
    n.rZ = 1.0 / (double)Z;
    return n;
}

// The pair scale of a chunk with scaled maxima mut, mud.  Where q vanishes
// on the chunk the unit is 0 (its min and residual are 0); where p does, c
// puts every draft exponent far below the target's (min(p, q) = 0 there).
__device__ __forceinline__ PairScale pair_scale(float mut, float mud, const RowNorm &t,
                                                const RowNorm &d) {
    PairScale ps;
    const float et = (mut > -kInf) ? __builtin_amdgcn_exp2f(mut - t.M) : 0.0f;
    const float ed = (mud > -kInf) ? __builtin_amdgcn_exp2f(mud - d.M) : 0.0f;
    const double at = (double)et * t.rZ, ad = (double)ed * d.rZ;
    ps.unit = (float)at;
    const double lk = !(at > 0.0) ? 1024.0 : !(ad > 0.0) ? -1024.0 : log2(ad / at);
    const double c = lk - (double)exp_ref(mud);
    ps.chi = (float)c;
    ps.clo = (float)(c - (double)ps.chi);
    return ps;
}

// min(p, q) of one element in units of alpha_t (see PairScale).
__device__ __forceinline__ float min_term(float zt, float zd, float s, float reft,
                                          const PairScale &ps) {
    const float a = __builtin_fmaf(zt, s, -reft);
    const float b = __builtin_fmaf(zd, s, ps.chi) + ps.clo;
    return __builtin_amdgcn_exp2f(__builtin_elementwise_minimum(a, b));
}

// Online combine of chunk statistics (scaled max mu, weight sum S) into a
// row's normalisers M = max mu and Z = sum S 2^(mu - M).  A NaN or +inf mu
// (a NaN or +inf logit in the chunk) makes M NaN.
struct OnlineZ {
    float m = -kInf;
    double z = 0.0;
    int bad = 0;
    __device__ __forceinline__ void add(float mu, float S) {
        if (!(mu == mu) || mu == kInf) {
            bad = 1;
        } else if (mu > -kInf) {
            if (mu > m) {
                z = __builtin_fma(z, (double)__builtin_amdgcn_exp2f(m - mu), (double)S);
                m = mu;
            } else {
                z = __builtin_fma((double)S, (double)__builtin_amdgcn_exp2f(mu - m), z);
            }
        }
    }
    // Wave-wide result (every lane gets it).
    __device__ __forceinline__ void reduce(float &M, float &Z) const {
        M = wave_max(m);
        const double zl = (m > -kInf) ? z * (double)__builtin_amdgcn_exp2f(m - M) : 0.0;
        Z = (float)wave_sum(zl);
        if (wave_max_i(bad)) M = __builtin_nanf("");
    }
};

// ---------------------------------------------------------------------------
// output helpers
// ---------------------------------------------------------------------------

// Invalid-request outputs of request r, written by the whole wave.
__device__ __forceinline__ void write_invalid(const VerifyArgs &a, int r) {
    const float nan = __builtin_nanf("");
    const int lane = lane_id();
    if (a.tv_mode) {
        if (lane == 0) {
            a.out_cs[r] = nan;
            if (a.out_rs) a.out_rs[r] = nan;
        }
    } else {
        for (int j = lane; j <= a.gamma; j += 64) {
            a.out_tok[(size_t)r * (a.gamma + 1) + j] = -1;
            if (a.out_lq) a.out_lq[(size_t)r * (a.gamma + 1) + j] = nan;
        }
        for (int i = lane; i < a.gamma; i += 64) {
            if (a.out_cs) a.out_cs[(size_t)r * a.gamma + i] = nan;
            if (a.out_rs) a.out_rs[(size_t)r * a.gamma + i] = nan;
        }
        if (lane == 0) a.out_n[r] = -1;
    }
    if (lane == 0) atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
}

// ---------------------------------------------------------------------------
// batched waits on tagged words
// ---------------------------------------------------------------------------

// A unit has at most kCB * 64 chunks, so a lane owns at most kCB of them
// (chunk c = 64 b + lane) and every per-chunk word of a unit fits in
// registers: the combines below issue all their loads at once and wait once.
constexpr int kCB = 4;

// Lane-parallel batch: word k of this lane is p[k] if act[k].  Issues every
// load, then re-reads only the words that do not carry `tag` yet, until all
// do.  out[k] = payload (0 for inactive words).  The wait is bounded: past
// kSpinLimit polls, or once any wave of the launch has timed out, it raises
// SPEC_DEV_SPIN_TIMEOUT and returns the stale payloads.
// `cached`: the words were written by an earlier launch, so a plain (cached)
// load sees them; only a stale tag (not expected) falls back to the coherent
// re-reads.
template <int K>
__device__ __forceinline__ void await_batch(const uint64_t *const (&p)[K], const bool (&act)[K],
                                            uint32_t tag, Control *ctl, uint32_t (&out)[K],
                                            bool cached = false) {
    uint64_t v[K];
    if (cached) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = act[k] ? *p[k] : ((uint64_t)tag << 32);
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = act[k] ? ld_word(p[k]) : ((uint64_t)tag << 32);
    }
    uint32_t it = 0;
    for (;;) {
        bool stale = false;
#pragma unroll
        for (int k = 0; k < K; ++k) stale = stale || (uint32_t)(v[k] >> 32) != tag;
        if (!__ballot(stale)) break;
        if ((++it & 255u) == 0u &&
            (it > kSpinLimit || (atomic_load_u32(&ctl->status) & SPEC_DEV_SPIN_TIMEOUT))) {
            if (stale) atomic_or_u32(&ctl->status, SPEC_DEV_SPIN_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int k = 0; k < K; ++k)
            if ((uint32_t)(v[k] >> 32) != tag) v[k] = ld_word(p[k]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) out[k] = (uint32_t)v[k];
}

// await_batch in two halves, so that other loads can be issued in between:
// words_issue loads every word unconditionally (an inactive one from `safe`,
// a valid address, and then reads as current), words_settle re-polls any
// stale active word.  Unconditional loads keep the compiler's wait counts
// exact for loads issued after them.
template <int K>
__device__ __forceinline__ void words_issue(const uint64_t *const (&p)[K], const bool (&act)[K],
                                            const uint64_t *safe, uint32_t tag,
                                            uint64_t (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint64_t w = *(act[k] ? p[k] : safe);
        v[k] = act[k] ? w : ((uint64_t)tag << 32);
    }
}
template <int K>
__device__ __forceinline__ void words_settle(const uint64_t *const (&p)[K], const bool (&act)[K],
                                             uint32_t tag, Control *ctl, uint64_t (&v)[K],
                                             uint32_t (&out)[K]) {
    uint32_t it = 0;
    for (;;) {
        bool stale = false;
#pragma unroll
        for (int k = 0; k < K; ++k) stale = stale || (act[k] && (uint32_t)(v[k] >> 32) != tag);
        if (!__ballot(stale)) break;
        if ((++it & 255u) == 0u &&
            (it > kSpinLimit || (atomic_load_u32(&ctl->status) & SPEC_DEV_SPIN_TIMEOUT))) {
            if (stale) atomic_or_u32(&ctl->status, SPEC_DEV_SPIN_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
        for (int k = 0; k < K; ++k)
            if (act[k] && (uint32_t)(v[k] >> 32) != tag) v[k] = ld_word(p[k]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) out[k] = (uint32_t)v[k];
}

// Chunk words of a unit, for the lane's chunks c = 64 (b0 + b) + lane
// (b < NB): w[b][q] = word q of chunk c (q < Q), 0 where c >= C or !want[q].
template <int Q, int NB = kCB>
__device__ __forceinline__ void load_unit_words(const uint64_t *base, int C, const bool (&want)[Q],
                                                uint32_t tag, Control *ctl,
                                                uint32_t (&w)[NB][Q], bool cached = false,
                                                int b0 = 0) {
    const uint64_t *p[NB * Q];
    bool act[NB * Q];
    uint32_t o[NB * Q];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int c = (b0 + b) * 64 + lane_id();
            p[b * Q + q] = base + (size_t)c * Q + q;
            act[b * Q + q] = c < C && want[q];
        }
    await_batch<NB * Q>(p, act, tag, ctl, o, cached);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < Q; ++q) w[b][q] = o[b * Q + q];
}

// ---------------------------------------------------------------------------
// inverse-CDF draw (two levels: chunk masses, then one chunk in id order)
// ---------------------------------------------------------------------------

// The chunk holding t in the running sum of the chunk masses m[b] (lane's
// chunks c = 64 b + lane, ascending chunk order, strict >).  Returns the chunk
// and, in *tin, t minus the mass before it; if t is at or past the total
// (rounding), the last chunk with mass and *tin = +inf.
__device__ __forceinline__ int select_chunk(int C, double t, const double (&m)[kCB], double *tin) {
    const int lane = lane_id();
    double run = 0.0;
    int clast = -1;
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
        const int c = b * 64 + lane;
        const double wc = (c < C) ? m[b] : 0.0;
        const double incl = wave_incl_scan_dpp(wc);
        const double excl = run + incl - wc;
        const uint64_t hit = __ballot(c < C && excl + wc > t);
        const uint64_t pos = __ballot(c < C && wc > 0.0);
        if (pos) clast = b * 64 + 63 - __builtin_clzll(pos);
        if (hit) {
            const int k = __builtin_ctzll(hit);
            *tin = readlane_d(t - excl, k);
            return b * 64 + k;
        }
        run += readlane_d(incl, 63);
    }
    *tin = INFINITY;
    return clast >= 0 ? clast : 0;
}

// Word q of chunk c from the lane-strided registers w (uniform result).
template <int Q>
__device__ __forceinline__ uint32_t chunk_word(const uint32_t (&w)[kCB][Q], int c, int q) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < kCB; ++b)
        if ((c >> 6) == b) v = rl(w[b][q], c & 63);
    return v;
}

// Draw inside chunk c0 of a row: the first id (ascending) whose running weight
// exceeds tin.  w[j][q] of lane l is the weight of id c0 + (64 j + l) EPV + q
// (0 past the row end).  Scans the chunk one vector row (64 lanes x EPV ids)
// at a time.  Clamps to the chunk's last positive weight; if none, its first
// id.
template <int N, int EPV>
__device__ __forceinline__ int draw_in_chunk_w(long c0, double tin,
                                               const float (&w)[N / EPV][EPV]) {
    const int lane = lane_id();
    double run = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int j = 0; j < N / EPV; ++j) {
        const long e = c0 + ((long)j * kLanes + lane) * EPV;
        double tot = 0.0;
        int lp = -1;
#pragma unroll
        for (int q = 0; q < EPV; ++q) {
            tot += (double)w[j][q];
            if (w[j][q] > 0.0f) lp = (int)e + q;
        }
        lastpos = max(lastpos, wave_max_i(lp));
        const double incl = wave_incl_scan_dpp(tot);
        const double excl = run + incl - tot;
        const uint64_t hit = __ballot(tot > 0.0 && excl + tot > tin);
        if (hit) {
            const int k = __builtin_ctzll(hit);
            int tok = -1;
            if (lane == k) {
                double cum = excl;
#pragma unroll
                for (int q = 0; q < EPV; ++q) {
                    cum += (double)w[j][q];
                    if (tok < 0 && cum > tin) tok = (int)e + q;
                }
                if (tok < 0) tok = lp;  // rounding: last positive id of this lane
            }
            return __builtin_amdgcn_readlane(tok, k);
        }
        run += readlane_d(incl, 63);
    }
    return lastpos >= 0 ? lastpos : (int)c0;
}

// Chunk logits in the draw's layout: z[j][q] of lane l is id c0 + (64 j + l)
// EPV + q; past the row end -inf.  The loads are unconditional (an id past
// the end re-reads id 0), so all of them are in flight at once.
template <typename T, int N, int EPV>
__device__ __forceinline__ void load_chunk_ids(const T *row, long c0, int V,
                                               float (&z)[N / EPV][EPV]) {
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < N / EPV; ++j) {
        const long e = c0 + ((long)j * kLanes + lane) * EPV;
        VecLoad<T, EPV>::run(row, e < V ? e : 0, z[j]);
        if (e >= V) {
#pragma unroll
            for (int q = 0; q < EPV; ++q) z[j][q] = -kInf;
        }
    }
}

// The logit of id tok (inside the chunk from c0) out of z, from its lane.
template <int N, int EPV>
__device__ __forceinline__ float chunk_logit(long c0, int tok, const float (&z)[N / EPV][EPV]) {
    const int rel = tok - (int)c0;
    const int jt = rel / (kLanes * EPV), lt = (rel / EPV) % kLanes, qt = rel % EPV;
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < N / EPV; ++j)
#pragma unroll
        for (int q = 0; q < EPV; ++q) v = (j == jt && q == qt) ? z[j][q] : v;
    return readlane_f(v, lt);
}

// ---------------------------------------------------------------------------
// unit folds (launch 2) and per-request combines (launch 3)
// ---------------------------------------------------------------------------

// The lane's chunk words of unit x (c = 64 b + lane), in rounds of two
// blocks in increasing chunk order, each handed to fold(w) for block
// b0 + h.  They come from the statistics pass (an earlier launch).
template <typename F>
__device__ __forceinline__ void fold_unit_words(const VerifyArgs &a, const Item &x, bool pair,
                                                F fold) {
    const int lane = lane_id();
    const bool want[4] = {true, true, pair, pair};
    for (int b0 = 0; b0 < kCB && b0 * 64 < a.C; b0 += 2) {
        uint32_t w[2][4];
        load_unit_words<4, 2>(a.st1 + (size_t)x.u * a.C * 4, a.C, want, a.tag, a.ctl, w, true,
                              b0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if ((b0 + h) * 64 + lane < a.C) fold(w[h]);
    }
}

__device__ __forceinline__ bool norms_ok(float M, float Z) {
    return finite_f(M) && Z > 0.0f && finite_f(Z);
}

// The accept test of a draft position (T > 0) on the gathered logits zx
// (target), dx (draft) of its draft token x_{i+1}, once the row normalisers
// are known: accept <=> q(x) >= p(x) or u < q(x)/p(x) (DART note eq. (3)), in
// fp64; *lqx = log q(x).  The uniform's range is checked by the combine.
__device__ __forceinline__ bool accept_eval(float zx, float dx, float s, float Mt, float Zt,
                                            float Md, float Zd, float uacc, float *lqx) {
    const double lq2 = (double)zx * (double)s - (double)Mt;
    const double lp2 = (double)dx * (double)s - (double)Md;
    const double q = exp2(lq2) / (double)Zt;
    const double pp = exp2(lp2) / (double)Zd;
    *lqx = (float)(lq2 * kLn2 - log((double)Zt));
    return q >= pp || (double)uacc < q / pp;
}

// The fold launch's work for draft position x at T > 0: its row normalisers
// M = max mu and Z = sum S 2^(mu - M) (per lane over its chunks in increasing
// order, then across the wave in a fixed order), each chunk's pair scale for
// the TV items --
// formed once here rather than in every TV item -- and the accept test, whose
// record (flags, log q(x)) the combine reads.  The draft token's two logits
// are gathered while the chunk words load.  The pair scales are published
// whatever the normalisers, so that the TV pass always finds current words;
// an invalid unit's TV sums are not used.
template <typename TT, typename TD>
__device__ __forceinline__ void norm_fold(const VerifyArgs &a, const Item &x, int xtok,
                                          float uacc) {
    const int lane = lane_id();
    const int C = a.C;
    float zx = 0.0f, dx = 0.0f;
    bool tok_ok = true;
    if (!a.tv_mode) {
        tok_ok = xtok >= 0 && xtok < a.V;
        if (tok_ok) {
            zx = load_one(row_ptr<TT>(a.zt, x.r, a.tG, x.i, a.V), xtok);
            dx = load_one(row_ptr<TD>(a.zd, x.r, a.dG, x.i, a.V), xtok);
        }
    }
    const bool want[4] = {true, true, true, true};
    uint32_t w[kCB][4];
    load_unit_words<4, kCB>(a.st1 + (size_t)x.u * C * 4, C, want, a.tag, a.ctl, w, true, 0);
    OnlineZ ot, od;
#pragma unroll
    for (int b = 0; b < kCB; ++b)
        if (b * 64 + lane < C) {
            ot.add(__uint_as_float(w[b][0]), __uint_as_float(w[b][1]));
            od.add(__uint_as_float(w[b][2]), __uint_as_float(w[b][3]));
        }
    float Mt, Zt, Md, Zd;
    ot.reduce(Mt, Zt);
    od.reduce(Md, Zd);
    publish_n(a.nrm + (size_t)x.u * 4, a.tag, 4, __float_as_uint(Mt), __float_as_uint(Zt),
              __float_as_uint(Md), __float_as_uint(Zd));
    const RowNorm nt = row_norm(Mt, Zt), nd = row_norm(Md, Zd);
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
        const int c = b * 64 + lane;
        if (c < C) {
            const PairScale ps =
                pair_scale(__uint_as_float(w[b][0]), __uint_as_float(w[b][2]), nt, nd);
            uint64_t *q = a.psc + ((size_t)x.u * C + c) * 4;
            st_word(q + 0, a.tag, __float_as_uint(ps.chi));
            st_word(q + 1, a.tag, __float_as_uint(ps.clo));
            st_word(q + 2, a.tag, __float_as_uint(ps.unit));
        }
    }
    if (!a.tv_mode) {
        const bool valid = norms_ok(Mt, Zt) && norms_ok(Md, Zd) && tok_ok;
        bool acc = false;
        float lqx = __builtin_nanf("");
        if (valid) acc = accept_eval(zx, dx, x.s, Mt, Zt, Md, Zd, uacc, &lqx);
        publish_n(a.rec + (size_t)x.u * kRecWords, a.tag, 2,
                  (valid ? kFlagValid : 0u) | (acc ? kFlagAccept : 0u), __float_as_uint(lqx),
                  0u, 0u);
    }
}

// Per-unit summary of a request in launch 3 (shared memory), written by
// lane 0 of the unit's wave.
struct UnitSum {
    uint32_t flags;          // kFlagValid, kFlagAccept
    float lqx;               // log q of the position's draft token (0 at T = 0)
    float cs, rs;            // c*, Res of a position
    int sel;                 // T = 0: the row's target argmax; T > 0: chunk of the
                             // inverse-CDF draw at this row (-1: no residual mass)
    float Mt, Zt, Md, Zd;    // row normalisers (T > 0)
    double tin;              // the draw's target minus the mass of chunks before sel
    double lnZt;             // ln Zt (T > 0), for the log q of a draw at this row
};

constexpr int kReqWaves = 8;
constexpr int kReqBlock = kReqWaves * 64;

// T = 0 unit (DART note sec. 2.3; survey sec. 1.3): the argmaxes of its rows
// (lowest id on ties); a position is accepted iff its draft token is the
// target argmax, and c* = [argmax p == argmax q].
__device__ __forceinline__ void greedy_unit(const VerifyArgs &a, const Item &x, UnitSum *s) {
    const bool pair = is_pair(x);
    int xtok = 0;
    if (!a.tv_mode && pair) xtok = a.tokens[(size_t)x.r * a.gamma + x.i];
    float vt = -kInf, vd = -kInf;
    int it = 0x7fffffff, id = 0x7fffffff, bad = 0;
    fold_unit_words(a, x, pair, [&](const uint32_t (&w)[4]) {
        if (w[1] == 0xffffffffu) bad = 1;
        else argmax_combine(vt, it, __uint_as_float(w[0]), (int)w[1]);
        if (pair) {
            if (w[3] == 0xffffffffu) bad = 1;
            else argmax_combine(vd, id, __uint_as_float(w[2]), (int)w[3]);
        }
    });
    wave_argmax(vt, it);
    wave_argmax(vd, id);
    bad = wave_max_i(bad);
    const int gt = (!bad && vt > -kInf && vt < kInf && it != 0x7fffffff) ? it : -1;
    const int gd = pair ? ((!bad && vd > -kInf && vd < kInf && id != 0x7fffffff) ? id : -1) : 0;
    bool valid = gt >= 0 && gd >= 0;
    bool acc = false;
    if (!a.tv_mode && pair) {
        valid = valid && xtok >= 0 && xtok < a.V;
        acc = xtok == gt;
    }
    if (lane_id() == 0) {
        const float cv = (gt == gd) ? 1.0f : 0.0f;
        s->flags = (valid ? kFlagValid : 0u) | (acc ? kFlagAccept : 0u);
        s->lqx = 0.0f;
        s->cs = pair ? cv : __builtin_nanf("");
        s->rs = pair ? 1.0f - cv : __builtin_nanf("");
        s->sel = gt;
    }
}

// T > 0 draft position: c* and Res from the TV pass's chunk words, the
// position's normalisers and accept record from the fold launch, and the
// chunk of the residual draw [q - p]_+ should this row be the request's first
// rejection (DART note eq. (3)-(4)).
__device__ __forceinline__ void tv_unit(const VerifyArgs &a, const Item &x, UnitSum *s) {
    const int lane = lane_id();
    const int C = a.C, G = a.gamma;
    float usm = 0.0f, uacc = 0.0f;
    if (!a.tv_mode) {
        usm = a.us[(size_t)x.r * (G + 1) + x.i];
        uacc = a.ua[(size_t)x.r * G + x.i];
    }
    const uint64_t *p[2 * kCB + 1];
    bool act[2 * kCB + 1];
    uint32_t o[2 * kCB + 1];
#pragma unroll
    for (int b = 0; b < kCB; ++b)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = b * 64 + lane;
            p[b * 2 + q] = a.st2 + ((size_t)x.u * C + c) * 2 + q;
            act[b * 2 + q] = c < C;
        }
    // lanes 0..3: normalisers; 4, 5: the fold's record (flags, log q(x))
    p[2 * kCB] = (lane < 4) ? a.nrm + (size_t)x.u * 4 + lane
                            : a.rec + (size_t)x.u * kRecWords + (lane & 1);
    act[2 * kCB] = lane < 4 || (!a.tv_mode && lane < 6);
    await_batch<2 * kCB + 1>(p, act, a.tag, a.ctl, o, true);
    const float Mt = __uint_as_float(rl(o[2 * kCB], 0)), Zt = __uint_as_float(rl(o[2 * kCB], 1));
    const float Md = __uint_as_float(rl(o[2 * kCB], 2)), Zd = __uint_as_float(rl(o[2 * kCB], 3));
    double cs = 0.0, rs = 0.0, m[kCB];
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
        cs += (double)__uint_as_float(o[b * 2]);
        m[b] = (double)__uint_as_float(o[b * 2 + 1]);
        rs += m[b];
    }
    cs = wave_sum(cs);
    rs = wave_sum(rs);
    bool valid, acc = false;
    float lqx = 0.0f;
    if (a.tv_mode) {
        valid = norms_ok(Mt, Zt) && norms_ok(Md, Zd);
    } else {
        const uint32_t fl = rl(o[2 * kCB], 4);
        lqx = __uint_as_float(rl(o[2 * kCB], 5));
        valid = (fl & kFlagValid) && uniform_ok(uacc) && uniform_ok(usm);
        acc = (fl & kFlagAccept) != 0;
    }
    int sel = -1;
    double tin = 0.0;
    if (valid && !a.tv_mode && rs > 0.0) sel = select_chunk(C, (double)usm * rs, m, &tin);
    if (lane == 0) {
        s->flags = (valid ? kFlagValid : 0u) | (acc ? kFlagAccept : 0u);
        s->lqx = lqx;
        s->cs = (float)cs;
        s->rs = (float)rs;
        s->sel = sel;
        s->Mt = Mt;
        s->Zt = Zt;
        s->Md = Md;
        s->Zd = Zd;
        s->tin = tin;
        s->lnZt = log((double)Zt);
    }
}

// T > 0 bonus unit (target row l_r): the row normalisers folded from the
// statistics words (per lane in increasing chunk order, then across the
// wave, as the fold launch folds a pair's), and the chunk of the
// inverse-CDF draw from q_l with u_sample[r][l] (DSpark guide, "basics": one
// bonus token).
__device__ __forceinline__ void bonus_unit(const VerifyArgs &a, const Item &x, UnitSum *s) {
    const int lane = lane_id();
    const int C = a.C;
    const float usm = a.us[(size_t)x.r * (a.gamma + 1) + x.i];
    const uint64_t *p[2 * kCB];
    bool act[2 * kCB];
    uint32_t o[2 * kCB];
#pragma unroll
    for (int b = 0; b < kCB; ++b)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = b * 64 + lane;
            p[b * 2 + q] = a.st1 + ((size_t)x.u * C + c) * 4 + q;
            act[b * 2 + q] = c < C;
        }
    await_batch<2 * kCB>(p, act, a.tag, a.ctl, o, true);
    OnlineZ ot;
#pragma unroll
    for (int b = 0; b < kCB; ++b)
        if (b * 64 + lane < C) ot.add(__uint_as_float(o[b * 2]), __uint_as_float(o[b * 2 + 1]));
    float Mt, Zt;
    ot.reduce(Mt, Zt);
    const bool valid = norms_ok(Mt, Zt) && uniform_ok(usm);
    int sel = -1;
    double tin = 0.0;
    if (valid) {
        double m[kCB];
        double W = 0.0;
#pragma unroll
        for (int b = 0; b < kCB; ++b) {
            const int c = b * 64 + lane;
            m[b] = (c < C) ? (double)chunk_alpha(__uint_as_float(o[b * 2]), Mt, Zt) *
                                 (double)__uint_as_float(o[b * 2 + 1])
                           : 0.0;
            W += m[b];
        }
        W = wave_sum(W);
        sel = select_chunk(C, (double)usm * W, m, &tin);
    }
    if (lane == 0) {
        s->flags = valid ? kFlagValid : 0u;
        s->lqx = 0.0f;
        s->cs = __builtin_nanf("");
        s->rs = __builtin_nanf("");
        s->sel = sel;
        s->Mt = Mt;
        s->Zt = Zt;
        s->Md = 0.0f;
        s->Zd = 1.0f;
        s->tin = tin;
        s->lnZt = log((double)Zt);
    }
}

// Draw inside chunk cs of target row trow from q: weights 2^(z s - mu) rebuilt
// exactly as the statistics pass made them, and the first id whose running
// weight exceeds tin (in probability units).  *ztok = the token's logit.
template <typename TT, int N, int EPV>
__device__ __forceinline__ int draw_q_chunk(const VerifyArgs &a, const TT *trow, int cs,
                                            double tin, float s, float mu, float M, float Z,
                                            float *ztok) {
    const float al = chunk_alpha(mu, M, Z);
    const float ref = exp_ref(mu);
    const long c0 = (long)cs * kLanes * N;
    const double te = (al > 0.0f) ? tin / (double)al : INFINITY;
    float z[N / EPV][EPV], wv[N / EPV][EPV];
    load_chunk_ids<TT, N, EPV>(trow, c0, a.V, z);
#pragma unroll
    for (int j = 0; j < N / EPV; ++j)
#pragma unroll
        for (int q = 0; q < EPV; ++q) wv[j][q] = ew(z[j][q], s, ref);
    const int tok = draw_in_chunk_w<N, EPV>(c0, te, wv);
    *ztok = chunk_logit<N, EPV>(c0, tok, z);
    return tok;
}

// Draw from q of a target row (T > 0), its chunk words w (mu_t, S_t in q = 0,
// 1) and normalisers (M, Z) in hand.  Returns the token; *ztok its logit.
template <typename TT, int N, int EPV, int Q>
__device__ __forceinline__ int draw_from_q(const VerifyArgs &a, const TT *trow,
                                           const uint32_t (&w)[kCB][Q], float s, float M, float Z,
                                           float uu, float *ztok) {
    const int C = a.C;
    double m[kCB];
    double W = 0.0;
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
        const int c = b * 64 + lane_id();
        m[b] = (c < C) ? (double)chunk_alpha(__uint_as_float(w[b][0]), M, Z) *
                             (double)__uint_as_float(w[b][1])
                       : 0.0;
        W += m[b];
    }
    W = wave_sum(W);
    double tin;
    const int cs = select_chunk(C, (double)uu * W, m, &tin);
    const float mu = __uint_as_float(chunk_word<Q>(w, cs, 0));
    return draw_q_chunk<TT, N, EPV>(a, trow, cs, tin, s, mu, M, Z, ztok);
}

// The request's committed draw at row j (T > 0), one wave: the residual draw
// from [q_j - p_j]_+ if j < l (DART note eq. (3)-(4); from q_j when that mass
// is exactly 0), else the bonus draw from q_l.  Returns the token; *lqd its
// log q.
template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ int request_draw(const VerifyArgs &a, int r, int j, int l, float s,
                                            const UnitSum &su, float *lqd) {
    const int lane = lane_id();
    const int C = a.C, G = a.gamma;
    const int u = r * a.UG + j;
    const float usm = a.us[(size_t)r * (G + 1) + j];
    const TT *trow = row_ptr<TT>(a.zt, r, a.tG, j, a.V);
    const float Mt = su.Mt, Zt = su.Zt;
    float ztok = 0.0f;
    int tok;
    if (j == l) {
        const uint64_t *const sp[1] = {a.st1 + ((size_t)u * C + su.sel) * 4};
        const bool sa[1] = {lane == 0};
        uint64_t sv[1];
        uint32_t so[1];
        words_issue<1>(sp, sa, sp[0], a.tag, sv);
        words_settle<1>(sp, sa, a.tag, a.ctl, sv, so);
        tok = draw_q_chunk<TT, N, EPV>(a, trow, su.sel, su.tin, s, __uint_as_float(rl(so[0], 0)),
                                       Mt, Zt, &ztok);
    } else if (su.sel >= 0) {
        // residual [q - p]_+: the chunk's words and both rows' logits in one
        // round of loads, then the chunk's weights in id order
        const TD *drow = row_ptr<TD>(a.zd, r, a.dG, j, a.V);
        const float Md = su.Md, Zd = su.Zd;
        const long c0 = (long)su.sel * kLanes * N;
        const uint64_t *const sp[1] = {a.st1 + ((size_t)u * C + su.sel) * 4 + (lane & 3)};
        const bool sa[1] = {lane < 4};
        uint64_t sv[1];
        uint32_t so[1];
        words_issue<1>(sp, sa, sp[0], a.tag, sv);
        float zt[N / EPV][EPV], zd[N / EPV][EPV];
        load_chunk_ids<TT, N, EPV>(trow, c0, a.V, zt);
        load_chunk_ids<TD, N, EPV>(drow, c0, a.V, zd);
        words_settle<1>(sp, sa, a.tag, a.ctl, sv, so);
        const float mut = __uint_as_float(rl(so[0], 0)), mud = __uint_as_float(rl(so[0], 2));
        const PairScale ps = pair_scale(mut, mud, row_norm(Mt, Zt), row_norm(Md, Zd));
        const float reft = exp_ref(mut);
        const double te = (ps.unit > 0.0f) ? su.tin / (double)ps.unit : INFINITY;
        float wv[N / EPV][EPV];
#pragma unroll
        for (int jj = 0; jj < N / EPV; ++jj)
#pragma unroll
            for (int q = 0; q < EPV; ++q) {
                // the TV pass's terms; the outer min keeps every weight >= 0
                const float et = ew(zt[jj][q], s, reft);
                const float mn = __builtin_elementwise_minimum(
                    et, min_term(zt[jj][q], zd[jj][q], s, reft, ps));
                wv[jj][q] = et - mn;
            }
        tok = draw_in_chunk_w<N, EPV>(c0, te, wv);
        ztok = chunk_logit<N, EPV>(c0, tok, zt);
    } else {
        // no residual mass (rounding): draw from q of the same row
        uint32_t w4[kCB][4];
        const bool want4[4] = {true, true, false, false};
        load_unit_words<4>(a.st1 + (size_t)u * C * 4, C, want4, a.tag, a.ctl, w4, true);
        tok = draw_from_q<TT, N, EPV, 4>(a, trow, w4, s, Mt, Zt, usm, &ztok);
    }
    *lqd = (float)(((double)ztok * (double)s - (double)Mt) * kLn2 - su.lnZt);
    return tok;
}

// Row-pair mode (spec_tv_accept_rate): one wave per pair writes c* and Res.
template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ void pair_combine(const VerifyArgs &a, int r, UnitSum *s) {
    Item x;
    x.u = r;
    x.r = r;
    x.i = 0;
    x.c = 0;
    x.l = 1;
    if (!request_ok(a, r, x.T, x.l)) {
        write_invalid(a, r);
        return;
    }
    x.s = x.T != 0.0f ? exp2_scale(x.T) : 0.0f;
    if (x.T == 0.0f) greedy_unit(a, x, s);
    else tv_unit(a, x, s);
    const uint32_t fl = __builtin_amdgcn_readfirstlane(s->flags);
    if (!(fl & kFlagValid)) {
        write_invalid(a, r);
    } else if (lane_id() == 0) {
        a.out_cs[r] = s->cs;
        if (a.out_rs) a.out_rs[r] = s->rs;
    }
}

// Launch 3.  Row-pair mode: one wave per pair.  Verification: one workgroup
// per request.  Its waves summarise units 0..l_r (accept flags, c*, Res and
// the chunk each row would draw from); then the first wave applies strict
// left-to-right prefix survival (DSpark guide, "basics": A_r = the number of
// leading accepts), makes the one draw the request commits (the residual at
// the first rejection, or the bonus from q_l; at T = 0 the target argmax of
// row A_r) and writes the request's outputs.  No state is shared across
// workgroups, and every word read was written by an earlier launch.
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kReqBlock) combine_kernel(VerifyArgs a) {
    a.tag = call_tag(a.ctl);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.ctl->tag_next = (a.tag + 1u) | 0x80000000u;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    __shared__ UnitSum sum[kMaxGamma + 1 > kReqWaves ? kMaxGamma + 1 : kReqWaves];
    if (a.tv_mode) {
        const int r = (int)blockIdx.x * kReqWaves + wave;
        if (r < a.R) pair_combine<TT, TD, N, EPV>(a, r, &sum[wave]);
        return;
    }
    const int r = blockIdx.x;
    // the draft tokens the outputs copy, loaded with the request's parameters
    // (wave 0 writes the outputs; lane k holds tokens k and 64 + k)
    int32_t dtok[2] = {0, 0};
    if (wave == 0) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
            if (b * 64 + lane < a.gamma) dtok[b] = a.tokens[(size_t)r * a.gamma + b * 64 + lane];
    }
    Item x;
    x.r = r;
    x.c = 0;
    if (!request_ok(a, r, x.T, x.l)) {
        if (wave == 0) write_invalid(a, r);
        return;
    }
    const int l = x.l, G = a.gamma;
    x.s = x.T != 0.0f ? exp2_scale(x.T) : 0.0f;
    for (int i = wave; i <= l; i += kReqWaves) {
        x.i = i;
        x.u = r * a.UG + i;
        if (x.T == 0.0f) greedy_unit(a, x, &sum[i]);
        else if (i < l) tv_unit(a, x, &sum[i]);
        else bonus_unit(a, x, &sum[i]);
    }
    __syncthreads();
    if (wave != 0) return;
    // prefix survival over the summaries (units 0..l sit on lanes 64 b + lane)
    bool bad = false, rej = false;
    int first_rej = 64 * 2;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int i = b * 64 + lane;
        const uint32_t fl = i <= l ? sum[i].flags : kFlagValid;
        bad = bad || !(fl & kFlagValid);
        rej = i < l && !(fl & kFlagAccept);
        const uint64_t m = __ballot(rej);
        if (m && first_rej == 128) first_rej = b * 64 + __builtin_ctzll(m);
    }
    if (__ballot(bad)) {
        write_invalid(a, r);
        return;
    }
    const int A = first_rej < l ? first_rej : l;
    int tok;
    float lqd;
    if (x.T == 0.0f) {
        tok = sum[A].sel;
        lqd = 0.0f;
    } else {
        tok = request_draw<TT, TD, N, EPV>(a, r, A, l, x.s, sum[A], &lqd);
    }
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int k = b * 64 + lane;
        if (k > G) break;
        const int32_t t = (k < A) ? dtok[b] : (k == A ? tok : -1);
        a.out_tok[(size_t)r * (G + 1) + k] = t;
        if (a.out_lq)
            a.out_lq[(size_t)r * (G + 1) + k] = (k < A) ? sum[k].lqx : (k == A ? lqd : nan);
        if (k < G) {
            if (a.out_cs) a.out_cs[(size_t)r * G + k] = (k < l) ? sum[k].cs : nan;
            if (a.out_rs) a.out_rs[(size_t)r * G + k] = (k < l) ? sum[k].rs : nan;
        }
    }
    if (lane == 0) a.out_n[r] = A;
}

// ---------------------------------------------------------------------------
// the four kernels
// ---------------------------------------------------------------------------

// Issues item x's loads: its chunk of the target row and, for a pair, of the
// draft row.
template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ void load_item(const VerifyArgs &a, const Item &x,
                                          RawChunk<TT, N, EPV> &rt, RawChunk<TD, N, EPV> &rd) {
    const long c0 = (long)x.c * kLanes * N;
    rt.load(row_ptr<TT>(a.zt, x.r, a.tG, x.i, a.V), c0, a.V);
    if (is_pair(x)) rd.load(row_ptr<TD>(a.zd, x.r, a.dG, x.i, a.V), c0, a.V);
}

// Stats of item x: the chunk words (mu, S) per row, or the argmax words at
// T = 0, published for the unit's combine and the TV pass.
template <int N, int EPV, typename RT, typename RD>
__device__ __forceinline__ void stats_item(const VerifyArgs &a, const Item &x, RT &rt, RD &rd) {
    const long c0 = (long)x.c * kLanes * N;
    rt.fix();
    if (is_pair(x)) rd.fix();
    uint32_t w0, w1, w2 = 0, w3 = 0;
    if (x.T == 0.0f) {
        float bv;
        int bi, bad;
        chunk_argmax<N, EPV>(rt, c0, bv, bi, bad);
        w0 = __float_as_uint(bv);
        w1 = bad ? 0xffffffffu : (uint32_t)bi;
        if (is_pair(x)) {
            chunk_argmax<N, EPV>(rd, c0, bv, bi, bad);
            w2 = __float_as_uint(bv);
            w3 = bad ? 0xffffffffu : (uint32_t)bi;
        }
    } else {
        float e[N], mu, S;
        chunk_exp<N>(rt, x.s, e, mu, S);
        w0 = __float_as_uint(mu);
        w1 = __float_as_uint(S);
        if (is_pair(x)) {
            chunk_exp<N>(rd, x.s, e, mu, S);
            w2 = __float_as_uint(mu);
            w3 = __float_as_uint(S);
        }
    }
    publish_all(a.st1 + ((size_t)x.u * a.C + x.c) * 4, a.tag, 4, w0, w1, w2, w3);
}

// Kernel 1: every needed row streamed once from HBM, one item in flight per
// wave (five waves per SIMD); per item the chunk words.
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kBlock, kStreamWaves) stats_kernel(VerifyArgs a) {
    a.tag = first_launch_tag(a.ctl);
    extern __shared__ uint32_t lds[];
    Walker cur = make_walker(a, lds, false);
    Item x;
    RawChunk<TT, N, EPV> rt;
    RawChunk<TD, N, EPV> rd;
    while (cur.next(a, x)) {
        load_item(a, x, rt, rd);
        stats_item<N, EPV>(a, x, rt, rd);
    }
}

// TV sums of one chunk pair at T > 0: with the chunk's words (mu_t, S_t,
// mu_d) and its pair scale, the weights e = 2^(z s - mu) are rebuilt exactly
// as the statistics made them; *cmin = the chunk's sum min(p, q) and
// *cres its residual mass sum [q - p]_+.  The logits must be fixed (past-the-
// row slots -inf).
template <int N, typename RT, typename RD>
__device__ __forceinline__ void tv_sums(const RT &rt, const RD &rd, float s, float mut, float St,
                                        const PairScale &ps, double *cmin, double *cres) {
    const float reft = exp_ref(mut);
    // min(p, q) in units of ps.unit, summed in the same slot order as the
    // chunk's weight sum St in the statistics pass, so a chunk with q <= p
    // everywhere has a residual of exactly 0
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < N; ++k) acc += min_term(rt.get(k), rd.get(k), s, reft, ps);
    const float smin = wave_sum_f(acc);
    *cmin = (double)ps.unit * (double)smin;
    *cres = fmax((double)ps.unit * ((double)St - (double)smin), 0.0);
}

// TV of pair item x at T > 0 (chunk re-read, from the Infinity Cache when the
// rows fit there), with the chunk's words and pair scale from the earlier
// launches (w8: lanes 0..3 the chunk's words, 4..6 its pair scale).
template <int N, typename RT, typename RD>
__device__ __forceinline__ void tv_item(const VerifyArgs &a, const Item &x, RT &rt, RD &rd,
                                        uint32_t w8) {
    rt.fix();
    rd.fix();
    double cmin, cres;
    PairScale ps;
    ps.chi = __uint_as_float(rl(w8, 4));
    ps.clo = __uint_as_float(rl(w8, 5));
    ps.unit = __uint_as_float(rl(w8, 6));
    tv_sums<N>(rt, rd, x.s, __uint_as_float(rl(w8, 0)), __uint_as_float(rl(w8, 1)), ps, &cmin,
               &cres);
    publish_all(a.st2 + ((size_t)x.u * a.C + x.c) * 2, a.tag, 2, __float_as_uint((float)cmin),
                __float_as_uint((float)cres), 0u, 0u);
}

// Issues the loads of pair item x: its chunk of both rows, and (lanes 0..6)
// the chunk's words and pair scale.
template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ uint64_t load_tv_item(const VerifyArgs &a, const Item &x,
                                                 RawChunk<TT, N, EPV> &rt,
                                                 RawChunk<TD, N, EPV> &rd) {
    const int lane = lane_id();
    const size_t ch = (size_t)x.u * a.C + x.c;
    const uint64_t *p = (lane < 4) ? a.st1 + ch * 4 + lane : a.psc + ch * 4 + (lane & 3);
    // plain loads: both kinds of word were written by earlier launches
    const uint64_t w = (lane < 7) ? *p : 0;
    load_item(a, x, rt, rd);
    return w;
}

// Kernel 2: one wave per draft position at T > 0 folds launch 1's chunk
// words into the position's row normalisers and each chunk's pair scale, and
// runs the accept test.
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kBlock) fold_kernel(VerifyArgs a) {
    a.tag = call_tag(a.ctl);
    const long u = wave_index();
    if (u >= (long)a.R * a.UG) return;
    Item y;
    y.u = (int)u;
    y.r = (int)(u / a.UG);
    y.i = (int)(u % a.UG);
    y.c = 0;
    // one round of loads: the request's parameters and the position's draft
    // token and uniform (read before the position is known to be verified;
    // they are in the arrays whenever i < gamma)
    y.T = a.temp[y.r];
    y.l = a.tv_mode ? 1 : a.vlen[y.r];
    int xtok = 0;
    float uacc = 0.0f;
    if (!a.tv_mode && y.i < a.gamma) {
        xtok = a.tokens[(size_t)y.r * a.gamma + y.i];
        uacc = a.ua[(size_t)y.r * a.gamma + y.i];
    }
    if (!temperature_ok(y.T) || y.l < 0 || y.l > a.gamma || y.T == 0.0f || !is_pair(y)) return;
    y.s = exp2_scale(y.T);
    norm_fold<TT, TD>(a, y, xtok, uacc);
}

// Kernel 3: the TV pass over the pair items at T > 0, one item in flight per
// wave.  Every word it reads is an earlier launch's, so no wave waits for
// another.
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kBlock, kStreamWaves) tv_kernel(VerifyArgs a) {
    a.tag = call_tag(a.ctl);
    const int lane = lane_id();
    extern __shared__ uint32_t lds[];
    Walker cur = make_walker(a, lds, true);
    Item x;
    RawChunk<TT, N, EPV> rt;
    RawChunk<TD, N, EPV> rd;
    while (cur.next(a, x)) {
        const uint64_t w = load_tv_item(a, x, rt, rd);
        // lanes 0..3: launch 1's chunk words, 4..6: launch 2's pair scale
        if (__ballot(lane < 7 && (uint32_t)(w >> 32) != a.tag) && lane == 0)
            atomic_or_u32(&a.ctl->status, SPEC_DEV_SPIN_TIMEOUT);
        tv_item<N>(a, x, rt, rd, (uint32_t)w);
    }
}

// ---------------------------------------------------------------------------
// held-pair path (bf16 rows): one launch does the statistics, the fold and
// the TV sums of every row pair at T > 0.  Each such pair belongs to one
// workgroup, which keeps most of its chunks on the compute unit between the
// two passes (registers, then shared memory) and reads only the rest again;
// the workgroups that hold no pair stream the other needed rows (bonus rows,
// T = 0 rows) for their statistics.  The combine launch follows unchanged.
// ---------------------------------------------------------------------------

constexpr int kHoldWaves = 8;                  // waves per workgroup (one workgroup per CU)
constexpr int kHoldBlock = kHoldWaves * 64;
constexpr int kHoldReg = 8;                   // chunk pairs per wave kept in registers
constexpr int kHoldFill = 8;                   // row chunks per filler batch (two in flight)
constexpr size_t kHoldLdsBytes = 160 * 1024;   // shared memory of a compute unit
constexpr size_t kHoldStaticLds = 1024;        // kept for the kernel's static shared memory

// Work list of the held path in shared memory: req[3 R] = (T, s, l), then the
// held pairs (r << 7 | i: positions i < l at T > 0), then the filler rows
// ((r << 7 | i) << 1 | row, row 1 = the draft row): every other row the
// statistics must cover (the bonus row at T > 0; every row at T = 0).
struct HoldTable {
    const uint32_t *req;
    const uint32_t *units;
    uint32_t held, filler;
};

__device__ __forceinline__ HoldTable build_hold_table(const VerifyArgs &a, uint32_t *lds) {
    __shared__ uint32_t wsum[kHoldWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t *req = lds;
    uint32_t *units = lds + 3 * a.R;
    const int K = (a.R + kHoldBlock - 1) / kHoldBlock;
    const int r0 = tid * K, r1 = min(r0 + K, a.R);
    // per-thread counts of held pairs (low half) and filler rows (high half);
    // both stay below 2^16 since the table fits the shared memory
    uint32_t own = 0;
    for (int r = r0; r < r1; ++r) {
        float T;
        int l;
        const bool ok = request_ok(a, r, T, l);
        req[3 * r + 0] = __float_as_uint(T);
        req[3 * r + 1] = __float_as_uint(ok && T != 0.0f ? exp2_scale(T) : 0.0f);
        req[3 * r + 2] = (uint32_t)l;
        const int n = table_units(a, ok, T, l, false);
        const int h = (ok && T != 0.0f) ? min(l, n) : 0;
        // filler units h..n-1: a draft row too for the pairs among them (i < l)
        const int fr = (n - h) + max(0, min(l, n) - h);
        own += (uint32_t)h + ((uint32_t)fr << 16);
    }
    const uint32_t incl = wave_incl_scan_dpp(own);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kHoldWaves; ++w) {
        if (w < wave) base += wsum[w];
        total += wsum[w];
    }
    const uint32_t ex = base + incl - own, held = total & 0xffffu;
    uint32_t ph = ex & 0xffffu, pf = held + (ex >> 16);
    for (int r = r0; r < r1; ++r) {
        const int l = (int)req[3 * r + 2];
        const float T = __uint_as_float(req[3 * r]);
        const bool ok = temperature_ok(T) && l >= 0 && l <= a.gamma;
        const int n = table_units(a, ok, T, l, false);
        const int h = (ok && T != 0.0f) ? min(l, n) : 0;
        for (int i = 0; i < h; ++i) units[ph++] = ((uint32_t)r << 7) | (uint32_t)i;
        for (int i = h; i < n; ++i) {
            const uint32_t e = (((uint32_t)r << 7) | (uint32_t)i) << 1;
            units[pf++] = e;
            if (i < l) units[pf++] = e | 1u;
        }
    }
    __syncthreads();
    HoldTable t;
    t.req = req;
    t.units = units;
    t.held = held;
    t.filler = total >> 16;
    return t;
}

// Shared memory of the held path: the table, a pair's chunk statistics
// (C x 4 floats), then kl slots of one chunk pair each (both rows' raw
// registers, lane-major: 2 x 8 words x 64 lanes).
__host__ __device__ constexpr size_t hold_slot_words() { return 2 * 8 * 64; }

// A chunk pair kept in shared-memory slot p: written after its statistics,
// read back for its TV sums.
template <typename RC>
__device__ __forceinline__ void slot_put(uint32_t *slots, int p, int row, const RC &rc) {
    uint32_t *d = slots + (size_t)p * hold_slot_words() + row * 512 + lane_id();
#pragma unroll
    for (int q = 0; q < 8; ++q) d[q * 64] = rc.w[q];
}
template <typename RC>
__device__ __forceinline__ void slot_get(const uint32_t *slots, int p, int row, RC &rc, long c0,
                                         int V) {
    const uint32_t *d = slots + (size_t)p * hold_slot_words() + row * 512 + lane_id();
#pragma unroll
    for (int q = 0; q < 8; ++q) rc.w[q] = d[q * 64];
    const long left = (long)V - c0;
    rc.rem = left < (long)kLanes * 16 ? (int)left : kLanes * 16;
}

// Statistics of chunk c of held pair x (both rows at T > 0): the chunk words
// for the combine's draws and the table entry for the fold.
template <int N, typename RC>
__device__ __forceinline__ void hold_stats(const VerifyArgs &a, const Item &x, int c, RC &rt,
                                           RC &rd, float *stt) {
    rt.fix();
    rd.fix();
    float e[N], mut, St, mud, Sd;
    chunk_exp<N>(rt, x.s, e, mut, St);
    chunk_exp<N>(rd, x.s, e, mud, Sd);
    if (lane_id() == 0) {
        stt[c * 4 + 0] = mut;
        stt[c * 4 + 1] = St;
        stt[c * 4 + 2] = mud;
        stt[c * 4 + 3] = Sd;
    }
    publish_all(a.st1 + ((size_t)x.u * a.C + c) * 4, a.tag, 4, __float_as_uint(mut),
              __float_as_uint(St), __float_as_uint(mud), __float_as_uint(Sd));
}

// TV sums of chunk c = w + 8 m of held pair x; lane m of the wave holds that
// chunk's words (mu_t, S_t) and pair scale.
template <int N, typename RC>
__device__ __forceinline__ void hold_tv(const VerifyArgs &a, const Item &x, int c, int m,
                                        RC &rt, RC &rd, float mut, float St,
                                        const PairScale &ps) {
    rt.fix();
    rd.fix();
    PairScale q;
    q.chi = rlf(ps.chi, m);
    q.clo = rlf(ps.clo, m);
    q.unit = rlf(ps.unit, m);
    double cmin, cres;
    tv_sums<N>(rt, rd, x.s, rlf(mut, m), rlf(St, m), q, &cmin, &cres);
    publish_all(a.st2 + ((size_t)x.u * a.C + c) * 2, a.tag, 2, __float_as_uint((float)cmin),
              __float_as_uint((float)cres), 0u, 0u);
}

// The next chunk of the pair's stream for the calling wave (a shared-memory
// counter, one claim per wave).
__device__ __forceinline__ int hold_claim(int *next) {
    int v = 0;
    if (lane_id() == 0)
        v = __hip_atomic_fetch_add(next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(v);
}

// One held pair x, the whole workgroup.  Wave w keeps chunks c = w + 8 m,
// m < kHoldReg, in registers; the later chunks are streamed by whichever wave
// claims them next from *next (which holds nreg + 8 on entry: each wave's
// first streamed chunk is nreg + w), so that every wave streams until the
// pair's last chunk; those that fit go to the shared-memory slots (chunk
// c to slot c - nreg), the rest are read again for the TV sums, where wave
// w takes the slot and re-read chunks c = w + 8 m.
template <int N, int EPV>
__device__ __forceinline__ void hold_pair(const VerifyArgs &a, const Item &x, float *stt,
                                          uint32_t *slots, int kl, int *next) {
    using RC = RawChunk<uint16_t, N, EPV>;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int C = a.C;
    const int nreg = kHoldWaves * kHoldReg;   // chunks kept in registers
    const int nlds = nreg + kl;                // ... and in shared memory
    const uint16_t *trow = row_ptr<uint16_t>(a.zt, x.r, a.tG, x.i, a.V);
    const uint16_t *drow = row_ptr<uint16_t>(a.zd, x.r, a.dG, x.i, a.V);
    // the accept test's token and uniform (wave 0)
    int xtok = 0;
    float uacc = 0.0f;
    if (w == 0 && !a.tv_mode) {
        xtok = a.tokens[(size_t)x.r * a.gamma + x.i];
        uacc = a.ua[(size_t)x.r * a.gamma + x.i];
    }
    // ---- pass 1: every chunk once, its statistics; most chunks kept.  A
    // chunk past the row's chunks re-reads chunk 0 (cached) and is not used.
    const long z0 = 0;
    RC ht[kHoldReg], hd[kHoldReg];
#pragma unroll
    for (int k = 0; k < kHoldReg; ++k) {
        const int c = w + kHoldWaves * k;
        const long c0 = c < C ? (long)c * kLanes * N : z0;
        ht[k].load(trow, c0, a.V);
        hd[k].load(drow, c0, a.V);
    }
    // the wave's first chunk past the registers, in flight behind them
    RC at, ad, bt, bd;
    int c = nreg + w;
    at.load(trow, c < C ? (long)c * kLanes * N : z0, a.V);
    ad.load(drow, c < C ? (long)c * kLanes * N : z0, a.V);
    float zx = 0.0f, dx = 0.0f;
    const bool tok_ok = xtok >= 0 && xtok < a.V;
    if (w == 0 && !a.tv_mode && tok_ok) {
        zx = load_one(trow, xtok);
        dx = load_one(drow, xtok);
    }
#pragma unroll
    for (int k = 0; k < kHoldReg; ++k) hold_stats<N>(a, x, w + kHoldWaves * k, ht[k], hd[k], stt);
    // the chunks past the registers, claimed one at a time, two in flight
    {
        int cb = hold_claim(next);
        while (c < C) {
            bt.load(trow, cb < C ? (long)cb * kLanes * N : z0, a.V);
            bd.load(drow, cb < C ? (long)cb * kLanes * N : z0, a.V);
            hold_stats<N>(a, x, c, at, ad, stt);
            if (c < nlds) {
                slot_put(slots, c - nreg, 0, at);
                slot_put(slots, c - nreg, 1, ad);
            }
            if (cb >= C) break;
            c = hold_claim(next);
            at.load(trow, c < C ? (long)c * kLanes * N : z0, a.V);
            ad.load(drow, c < C ? (long)c * kLanes * N : z0, a.V);
            hold_stats<N>(a, x, cb, bt, bd, stt);
            if (cb < nlds) {
                slot_put(slots, cb - nreg, 0, bt);
                slot_put(slots, cb - nreg, 1, bd);
            }
            cb = hold_claim(next);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) *next = nreg + kHoldWaves;  // for the next pair's stream
    // ---- the fold, in every wave (fixed order: the same bits everywhere) ----
    OnlineZ ot, od;
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
        const int c = b * 64 + lane;
        if (c < C) {
            ot.add(stt[c * 4 + 0], stt[c * 4 + 1]);
            od.add(stt[c * 4 + 2], stt[c * 4 + 3]);
        }
    }
    float Mt, Zt, Md, Zd;
    ot.reduce(Mt, Zt);
    od.reduce(Md, Zd);
    if (w == 0) {
        publish_n(a.nrm + (size_t)x.u * 4, a.tag, 4, __float_as_uint(Mt), __float_as_uint(Zt),
                  __float_as_uint(Md), __float_as_uint(Zd));
        if (!a.tv_mode) {
            const bool valid = norms_ok(Mt, Zt) && norms_ok(Md, Zd) && tok_ok;
            bool acc = false;
            float lqx = __builtin_nanf("");
            if (valid) acc = accept_eval(zx, dx, x.s, Mt, Zt, Md, Zd, uacc, &lqx);
            publish_n(a.rec + (size_t)x.u * kRecWords, a.tag, 2,
                      (valid ? kFlagValid : 0u) | (acc ? kFlagAccept : 0u), __float_as_uint(lqx),
                      0u, 0u);
        }
    }
    // lane m: words and pair scale of the wave's chunk w + 8 m
    const int cm = w + kHoldWaves * lane;
    float mut = 0.0f, St = 0.0f;
    PairScale ps;
    ps.unit = ps.chi = ps.clo = 0.0f;
    if (cm < C) {
        mut = stt[cm * 4 + 0];
        St = stt[cm * 4 + 1];
        ps = pair_scale(mut, stt[cm * 4 + 2], row_norm(Mt, Zt), row_norm(Md, Zd));
    }
    // ---- pass 2: TV sums; the chunks past the slots are read again first ----
    {
        // the wave's first chunk past the slots
        c = nreg + w;
        while (c < nlds) c += kHoldWaves;
        at.load(trow, c < C ? (long)c * kLanes * N : z0, a.V);
        ad.load(drow, c < C ? (long)c * kLanes * N : z0, a.V);
#pragma unroll
        for (int k = 0; k < kHoldReg; ++k)
            hold_tv<N>(a, x, w + kHoldWaves * k, k, ht[k], hd[k], mut, St, ps);
        for (int cs = nreg + w; cs < C && cs < nlds; cs += kHoldWaves) {
            const long c0 = (long)cs * kLanes * N;
            RC st, sd;
            slot_get(slots, cs - nreg, 0, st, c0, a.V);
            slot_get(slots, cs - nreg, 1, sd, c0, a.V);
            hold_tv<N>(a, x, cs, (cs - w) / kHoldWaves, st, sd, mut, St, ps);
        }
        for (; c < C; c += 2 * kHoldWaves) {
            const int cb = c + kHoldWaves, cn = c + 2 * kHoldWaves;
            bt.load(trow, cb < C ? (long)cb * kLanes * N : z0, a.V);
            bd.load(drow, cb < C ? (long)cb * kLanes * N : z0, a.V);
            hold_tv<N>(a, x, c, (c - w) / kHoldWaves, at, ad, mut, St, ps);
            if (cb >= C) break;
            at.load(trow, cn < C ? (long)cn * kLanes * N : z0, a.V);
            ad.load(drow, cn < C ? (long)cn * kLanes * N : z0, a.V);
            hold_tv<N>(a, x, cb, (cb - w) / kHoldWaves, bt, bd, mut, St, ps);
        }
    }
    __syncthreads();  // the table entries and slots are reused by the next pair
}

// Filler row item k of the table: its unit (r, i), which row, which chunk.
struct FillItem {
    Item x;
    int row;
    const uint16_t *ptr;
    long c0;
};
__device__ __forceinline__ FillItem fill_item(const VerifyArgs &a, const HoldTable &t, uint32_t k,
                                              int N) {
    FillItem f;
    const uint32_t U = k / (uint32_t)a.C;
    f.x.c = (int)(k - U * (uint32_t)a.C);
    const uint32_t e = __builtin_amdgcn_readfirstlane(t.units[t.held + U]);
    f.row = (int)(e & 1u);
    f.x.r = (int)(e >> 8);
    f.x.i = (int)((e >> 1) & 127u);
    f.x.T = __uint_as_float(__builtin_amdgcn_readfirstlane(t.req[3 * f.x.r]));
    f.x.s = __uint_as_float(__builtin_amdgcn_readfirstlane(t.req[3 * f.x.r + 1]));
    f.x.l = (int)__builtin_amdgcn_readfirstlane(t.req[3 * f.x.r + 2]);
    f.x.u = f.x.r * a.UG + f.x.i;
    f.ptr = f.row ? row_ptr<uint16_t>(a.zd, f.x.r, a.dG, f.x.i, a.V)
                  : row_ptr<uint16_t>(a.zt, f.x.r, a.tG, f.x.i, a.V);
    f.c0 = (long)f.x.c * kLanes * N;
    return f;
}

// Statistics of one filler row chunk: (mu, S) at T > 0, the argmax words at
// T = 0, as the row's half of the chunk's four words.
template <int N, int EPV, typename RC>
__device__ __forceinline__ void fill_stats(const VerifyArgs &a, const FillItem &f, RC &rc) {
    rc.fix();
    uint32_t w0, w1;
    if (f.x.T == 0.0f) {
        float bv;
        int bi, bad;
        chunk_argmax<N, EPV>(rc, f.c0, bv, bi, bad);
        w0 = __float_as_uint(bv);
        w1 = bad ? 0xffffffffu : (uint32_t)bi;
    } else {
        float e[N], mu, S;
        chunk_exp<N>(rc, f.x.s, e, mu, S);
        w0 = __float_as_uint(mu);
        w1 = __float_as_uint(S);
    }
    publish_n(a.st1 + ((size_t)f.x.u * a.C + f.x.c) * 4 + 2 * f.row, a.tag, 2, w0, w1, 0u, 0u);
}

// The filler row items [lo, hi) of this workgroup, item lo + w + 8 j to wave
// w, in batches of kHoldFill with the next batch in flight.  Loads past hi
// re-read item lo's chunk (cached) and are not used.
template <int N, int EPV>
__device__ __forceinline__ void hold_fill(const VerifyArgs &a, const HoldTable &t, uint32_t lo,
                                          uint32_t hi) {
    using RC = RawChunk<uint16_t, N, EPV>;
    const uint32_t w = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (lo >= hi) return;
    const FillItem f0 = fill_item(a, t, lo, N);
    RC A[kHoldFill], B[kHoldFill];
    auto issue = [&](RC (&X)[kHoldFill], uint32_t k0) {
#pragma unroll
        for (int j = 0; j < kHoldFill; ++j) {
            const uint32_t k = k0 + (uint32_t)j * kHoldWaves;
            if (k < hi) {
                const FillItem f = fill_item(a, t, k, N);
                X[j].load(f.ptr, f.c0, a.V);
            } else {
                X[j].load(f0.ptr, f0.c0, a.V);
            }
        }
    };
    auto process = [&](RC (&X)[kHoldFill], uint32_t k0) {
#pragma unroll
        for (int j = 0; j < kHoldFill; ++j) {
            const uint32_t k = k0 + (uint32_t)j * kHoldWaves;
            if (k < hi) fill_stats<N, EPV>(a, fill_item(a, t, k, N), X[j]);
        }
    };
    const uint32_t step = kHoldFill * kHoldWaves;
    uint32_t k = lo + w;
    issue(A, k);
    for (; k < hi; k += 2 * step) {
        issue(B, k + step);
        process(A, k);
        if (k + step >= hi) break;
        issue(A, k + 2 * step);
        process(B, k + step);
    }
}

// The held-path launch: workgroup g holds pairs g, g + G, ... in turn; the
// workgroups with one pair fewer than the most loaded share the filler rows.
template <int N, int EPV>
__global__ void __launch_bounds__(kHoldBlock, 1) hold_kernel(VerifyArgs a, int kl) {
    a.tag = first_launch_tag(a.ctl);
    extern __shared__ uint32_t lds[];
    __shared__ int next;  // the held pairs' stream counter
    if (threadIdx.x == 0) next = kHoldWaves * kHoldReg + kHoldWaves;
    const HoldTable t = build_hold_table(a, lds);
    const size_t tw = 3 * (size_t)a.R + (size_t)t.held + t.filler;
    float *stt = (float *)(lds + ((tw + 3) & ~(size_t)3));
    uint32_t *slots = (uint32_t *)(stt + 4 * (size_t)a.C);
    const uint32_t G = gridDim.x, g = blockIdx.x;
    for (uint32_t k = g; k < t.held; k += G) {
        Item x;
        const uint32_t e = t.units[k];
        x.r = (int)(e >> 7);
        x.i = (int)(e & 127u);
        x.c = 0;
        x.T = __uint_as_float(t.req[3 * x.r]);
        x.s = __uint_as_float(t.req[3 * x.r + 1]);
        x.l = (int)t.req[3 * x.r + 2];
        x.u = x.r * a.UG + x.i;
        hold_pair<N, EPV>(a, x, stt, slots, kl, &next);
    }
    // filler rows: pairs in the last round P' = held - (rounds - 1) G; the
    // workgroups past P' (all, when P' = G) share them evenly
    const uint32_t rounds = (t.held + G - 1) / G;
    const uint32_t last = t.held - (rounds ? rounds - 1 : 0) * G;
    const uint32_t L = (rounds && last < G) ? G - last : G;
    if (rounds && last < G && g < last) return;
    const uint32_t li = (rounds && last < G) ? g - last : g;
    const uint64_t F = (uint64_t)t.filler * a.C;
    hold_fill<N, EPV>(a, t, (uint32_t)(F * li / L), (uint32_t)(F * (li + 1) / L));
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

struct Plan {
    int N;           // logits per lane per row
    int C;           // chunks per row
    long units;
    // tagged words after the control block
    size_t off_st1, off_st2, off_nrm, off_rec, off_psc, bytes;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// kN logits per lane and row: the weights of both rows then stay in registers
// at four waves per SIMD.
constexpr int kN = 16;

bool make_plan(long R, long units_per_req, long V, Plan &p) {
    const int N = kN;
    const long C = (V + (long)kLanes * N - 1) / ((long)kLanes * N);
    if (C > kCB * 64) return false;  // the combines hold a unit's chunk words in registers
    const long units = R * units_per_req;
    if (units * C > 0x7fffffffL) return false;
    p.N = N;
    p.C = (int)C;
    p.units = units;
    p.off_st1 = round_up(sizeof(Control), 256);
    p.off_st2 = round_up(p.off_st1 + 32 * (size_t)units * C, 256);
    p.off_nrm = round_up(p.off_st2 + 16 * (size_t)units * C, 256);
    p.off_rec = round_up(p.off_nrm + 32 * (size_t)units, 256);
    p.off_psc = round_up(p.off_rec + 8 * kRecWords * (size_t)units, 256);
    p.bytes = round_up(p.off_psc + 32 * (size_t)units * C, 256);
    return true;
}

size_t plan_bytes(long R, long upr, long V) {
    Plan p;
    return make_plan(R, upr, V, p) ? p.bytes : 0;
}

bool dtype_ok(int d) { return d == SPEC_F32 || d == SPEC_BF16; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Host-side caches of occupancy queries and compute-unit counts: fixed tables
// of plain values behind a spin lock, so that no call allocates host memory
// and nothing needs destroying when the process exits.
constexpr int kMaxDevices = 64;
constexpr int kOccSlots = 512;
struct OccEntry {
    const void *k;
    int dev;
    size_t lds;
    long cap;
};
OccEntry g_occ[kOccSlots];
int g_occ_n = 0;
std::atomic_flag g_occ_lock = ATOMIC_FLAG_INIT;
std::atomic<int> g_cus[kMaxDevices];

struct SpinGuard {
    std::atomic_flag &f;
    explicit SpinGuard(std::atomic_flag &flag) : f(flag) {
        while (f.test_and_set(std::memory_order_acquire)) {
        }
    }
    ~SpinGuard() { f.clear(std::memory_order_release); }
};

// Resident workgroups of `kernel` (kBlock threads, `lds` bytes of dynamic
// shared memory) on the whole current device, 0 if unknown.
long resident_blocks(const void *kernel, size_t lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    {
        SpinGuard g(g_occ_lock);
        for (int e = 0; e < g_occ_n; ++e)
            if (g_occ[e].k == kernel && g_occ[e].dev == dev && g_occ[e].lds == lds)
                return g_occ[e].cap;
    }
    int nb = 0, ncu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kBlock, lds) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const long cap = (long)nb * ncu;
    SpinGuard g(g_occ_lock);
    if (g_occ_n < kOccSlots) g_occ[g_occ_n++] = OccEntry{kernel, dev, lds, cap};
    return cap;
}

// Compute units of the current device (cached per device; 0 if unknown).
long device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(ncu, std::memory_order_relaxed);
    return ncu;
}

// Persistent grid of kernel k: its resident capacity, at most kStreamWaves
// workgroups per CU (the streaming passes measure fastest there, also when
// the registers would let more be resident), at most one wave per item.
long persistent_grid(const void *k, size_t lds, long items) {
    long cap = resident_blocks(k, lds);
    const long cus = device_cus();
    if (cap > 0 && cus > 0 && cap > cus * kStreamWaves) cap = cus * kStreamWaves;
    const long want = (items + kWaves - 1) / kWaves;
    if (cap <= 0) return want > 0 ? want : 1;
    const long g = want < cap ? want : cap;
    return g > 0 ? g : 1;
}

// Events recorded around the statistics launch of the calling thread's next
// verification calls (spec_time_stats_launch).
struct StatsTiming {
    void *const *before;
    void *const *after;
    int n, i;
};
thread_local StatsTiming g_stats_timing = {nullptr, nullptr, 0, 0};

// Shared memory of the unit table (0: too large, walk all candidates).
constexpr size_t kMaxTableBytes = 32768;
size_t table_bytes(const VerifyArgs &a) {
    const size_t b = 4 * (3 * (size_t)a.R + (size_t)a.R * a.UG);
    return b <= kMaxTableBytes ? (b + 255) / 256 * 256 : 0;
}

// Shared memory of the held path, 0 where it does not apply: the work list,
// one pair's chunk statistics and as many chunk-pair slots as fit (*kl).
size_t hold_bytes(const VerifyArgs &a, int *kl) {
    const size_t tw = 3 * (size_t)a.R + (size_t)a.R * (a.UG + a.gamma);
    const size_t head = ((tw + 3) & ~(size_t)3) * 4 + 16 * (size_t)a.C;
    const size_t cap = kHoldLdsBytes - kHoldStaticLds;
    if (4 * tw > kMaxTableBytes || head > cap) return 0;
    const long room = (long)((cap - head) / (hold_slot_words() * 4));
    const long need = (long)a.C - kHoldWaves * kHoldReg;
    if (need < 1) return 0;  // every register chunk exists and is whole
    const long n = need < room ? need : room;
    *kl = (int)n;
    return head + (size_t)n * hold_slot_words() * 4;
}

// Whether a call of this shape takes the held path on the current device
// (bf16 rows in 16-byte vectors assumed): its shared memory fits, every
// register chunk is whole (more than kHoldWaves * kHoldReg chunks), and at
// most two rounds of pairs fall to a workgroup even when every position is
// verified (larger batches stream faster through the split path).
// SPECVERIFY_SPLIT=1 in the environment selects the split path.
bool hold_applies(const VerifyArgs &a, int *kl, size_t *lds, long *G) {
    *lds = hold_bytes(a, kl);
    *G = device_cus();
    if (*lds == 0 || *G <= 0) return false;
    if ((long)a.R * (a.tv_mode ? 1 : (a.gamma > 0 ? a.gamma : 1)) > 2 * *G) return false;
    const char *sp = getenv("SPECVERIFY_SPLIT");
    return !(sp && sp[0] == '1');
}

// The held path for bf16 rows: one launch for the statistics, folds and TV
// sums, then the combine.  Returns -1 when it does not apply (the split path
// runs instead), else the launch status.
template <int N, int EPV>
int launch_hold(VerifyArgs a, hipStream_t st) {
    if constexpr (N != 16 || EPV != 8) {
        return -1;
    } else {
        int kl = 0;
        size_t lds = 0;
        long G = 0;
        if (!hold_applies(a, &kl, &lds, &G)) return -1;
        const void *k = reinterpret_cast<const void *>(&hold_kernel<N, EPV>);
        static std::atomic<int> attr{0};
        if (attr.load(std::memory_order_relaxed) == 0) {
            if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)(kHoldLdsBytes - kHoldStaticLds)) != hipSuccess)
                return -1;
            attr.store(1, std::memory_order_relaxed);
        }
        const long gc = a.tv_mode ? (a.R + kReqWaves - 1) / kReqWaves : a.R;
        a.tag = 0;
        StatsTiming &tm = g_stats_timing;
        const bool timed = tm.i < tm.n;
        if (timed) (void)hipEventRecord((hipEvent_t)tm.before[tm.i], st);
        hipLaunchKernelGGL((hold_kernel<N, EPV>), dim3((unsigned)G), dim3(kHoldBlock), lds, st, a,
                           kl);
        if (timed) (void)hipEventRecord((hipEvent_t)tm.after[tm.i++], st);
        hipLaunchKernelGGL((combine_kernel<uint16_t, uint16_t, N, EPV>), dim3((unsigned)gc),
                           dim3(kReqBlock), 0, st, a);
        return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
    }
}

template <typename TT, typename TD, int N, int EPV>
int launch_kernels(VerifyArgs a, hipStream_t st) {
    if constexpr (std::is_same<TT, uint16_t>::value && std::is_same<TD, uint16_t>::value) {
        const int h = launch_hold<N, EPV>(a, st);
        if (h >= 0) return h;
    }
    const void *k1 = reinterpret_cast<const void *>(&stats_kernel<TT, TD, N, EPV>);
    const void *k3 = reinterpret_cast<const void *>(&tv_kernel<TT, TD, N, EPV>);
    const long gf = ((long)a.R * a.UG + kWaves - 1) / kWaves;
    const size_t lds = table_bytes(a);
    a.compact = lds > 0;
    const long items = (long)a.R * a.UG * a.C;
    const long g1 = persistent_grid(k1, lds, items), g3 = persistent_grid(k3, lds, items);
    const long gc = a.tv_mode ? (a.R + kReqWaves - 1) / kReqWaves : a.R;
    a.tag = 0;  // read on the device by every launch
    static bool said = false;
    if (!said && getenv("SPECVERIFY_VERBOSE")) {
        said = true;
        fprintf(stderr, "[specverify] verify N=%d EPV=%d C=%d items=%ld grids %ld / %ld lds %zu\n",
                N, EPV, a.C, items, g1, g3, lds);
    }
    StatsTiming &tm = g_stats_timing;
    const bool timed = tm.i < tm.n;
    if (timed) (void)hipEventRecord((hipEvent_t)tm.before[tm.i], st);
    hipLaunchKernelGGL((stats_kernel<TT, TD, N, EPV>), dim3((unsigned)g1), dim3(kBlock), lds, st,
                       a);
    if (timed) (void)hipEventRecord((hipEvent_t)tm.after[tm.i++], st);
    hipLaunchKernelGGL((fold_kernel<TT, TD, N, EPV>), dim3((unsigned)gf), dim3(kBlock), 0, st, a);
    hipLaunchKernelGGL((tv_kernel<TT, TD, N, EPV>), dim3((unsigned)g3), dim3(kBlock), lds, st, a);
    hipLaunchKernelGGL((combine_kernel<TT, TD, N, EPV>), dim3((unsigned)gc), dim3(kReqBlock), 0,
                       st, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

template <typename TT, typename TD, int N>
int launch_n(const VerifyArgs &a, bool vec, hipStream_t st) {
    constexpr int ev = ChunkGeom<TT, TD, N>::kVec;
    return vec ? launch_kernels<TT, TD, N, ev>(a, st) : launch_kernels<TT, TD, N, 1>(a, st);
}

template <typename TT, typename TD>
int launch_types(const VerifyArgs &a, int N, bool vec, hipStream_t st) {
    if (N == kN) return launch_n<TT, TD, kN>(a, vec, st);
    return SPEC_EUNSUPPORTED;
}

int launch(const VerifyArgs &a, int tdt, int ddt, int N, bool vec, hipStream_t st) {
    if (tdt == SPEC_BF16 && ddt == SPEC_BF16) return launch_types<uint16_t, uint16_t>(a, N, vec, st);
    if (tdt == SPEC_F32 && ddt == SPEC_F32) return launch_types<float, float>(a, N, vec, st);
    if (tdt == SPEC_BF16 && ddt == SPEC_F32) return launch_types<uint16_t, float>(a, N, vec, st);
    return launch_types<float, uint16_t>(a, N, vec, st);
}

void bind_workspace(VerifyArgs &a, void *ws, const Plan &p) {
    char *b = (char *)ws;
    a.ctl = (Control *)b;
    a.st1 = (uint64_t *)(b + p.off_st1);
    a.st2 = (uint64_t *)(b + p.off_st2);
    a.nrm = (uint64_t *)(b + p.off_nrm);
    a.rec = (uint64_t *)(b + p.off_rec);
    a.psc = (uint64_t *)(b + p.off_psc);
    a.C = p.C;
}

}  // namespace
}  // namespace sv

using namespace sv;

// Workspace of spec_verify_batch_noalloc: one copy per device, zero-filled
// when the code object is loaded, held until the process ends.  Host code
// never passes this name to a kernel (on the host it only stands for the
// symbol): it uses the device address hipGetSymbolAddress gives for it.
static __device__ __align__(256) uint8_t scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {
// Device address of `scratch` per device, taken on the first call there.
std::atomic<void *> g_scratch_ptr[sv::kMaxDevices];

int scratch_ptr(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= sv::kMaxDevices) return SPEC_EHIP;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // the current device is `dev`: its copy of the array
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPEC_EHIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return SPEC_OK;
}
}  // namespace

extern "C" {

int spec_version(void) { return 200; }

const char *spec_status_string(int status) {
    switch (status) {
        case SPEC_OK: return "SPEC_OK";
        case SPEC_EINVAL: return "SPEC_EINVAL: null required pointer or invalid size";
        case SPEC_EDTYPE: return "SPEC_EDTYPE: unsupported dtype";
        case SPEC_EWORKSPACE: return "SPEC_EWORKSPACE: workspace null, too small or misaligned";
        case SPEC_EHIP: return "SPEC_EHIP: HIP runtime call or kernel launch failed";
        case SPEC_EUNSUPPORTED: return "SPEC_EUNSUPPORTED: shape outside the supported range";
        case SPEC_ETOOLARGE:
            return "SPEC_ETOOLARGE: the call needs more workspace than the no-allocation "
                   "entry point's fixed scratch holds";
    }
    return "unknown spec_status";
}

size_t spec_verify_workspace_bytes(int R, int gamma, int V) {
    if (R < 0 || gamma < 0 || gamma > kMaxGamma || V < 1 || V > SPEC_MAX_VERIFY_VOCAB) return 0;
    return plan_bytes(R > 0 ? R : 1, gamma + 1, V);
}

size_t spec_tv_workspace_bytes(int N, int V) {
    if (N < 0 || V < 1 || V > SPEC_MAX_VERIFY_VOCAB) return 0;
    return plan_bytes(N > 0 ? N : 1, 1, V);
}

int spec_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace || workspace_bytes < sizeof(Control) || ((uintptr_t)workspace & 255u))
        return SPEC_EWORKSPACE;
    const size_t words = workspace_bytes / 4;
    const size_t blocks = (words + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                       dim3(kBlock), 0, (hipStream_t)stream, (uint32_t *)workspace, words);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

int spec_time_stats_launch(void *const *before, void *const *after, int n) {
    if (n < 0 || (n > 0 && (!before || !after))) return SPEC_EINVAL;
    g_stats_timing = StatsTiming{before, after, n, 0};
    return SPEC_OK;
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
    if (gamma > kMaxGamma || V > SPEC_MAX_VERIFY_VOCAB) return SPEC_EUNSUPPORTED;
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
    // with gamma == 0 no draft row exists; the draft type only shapes the plan
    const int ddt = gamma > 0 ? d_dtype : t_dtype;
    return launch(a, t_dtype, ddt, p.N, vec, (hipStream_t)stream);
}

int spec_verify_batch_noalloc(const void *target_logits, int t_dtype, const void *draft_logits,
                              int d_dtype, const int32_t *draft_tokens,
                              const int32_t *verify_len, const float *temperature,
                              const float *u_accept, const float *u_sample, int R, int gamma,
                              int V, int32_t *out_tokens, int32_t *out_num_accepted,
                              float *out_cstar, float *out_resid_mass, float *out_logq,
                              void *stream) {
    if (R < 0 || gamma < 0 || V < 1) return SPEC_EINVAL;
    if (gamma > kMaxGamma || V > SPEC_MAX_VERIFY_VOCAB) return SPEC_EUNSUPPORTED;
    if (R == 0) return SPEC_OK;
    const size_t need = spec_verify_workspace_bytes(R, gamma, V);
    if (need == 0) return SPEC_EUNSUPPORTED;
    if (need > (size_t)SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_ETOOLARGE;
    void *ws = nullptr;
    const int st = scratch_ptr(&ws);
    if (st != SPEC_OK) return st;
    return spec_verify_batch(target_logits, t_dtype, draft_logits, d_dtype, draft_tokens,
                             verify_len, temperature, u_accept, u_sample, R, gamma, V, out_tokens,
                             out_num_accepted, out_cstar, out_resid_mass, out_logq, ws,
                             (size_t)SPEC_NOALLOC_SCRATCH_BYTES, stream);
}

int spec_verify_path(int R, int gamma, int V, int t_dtype, int d_dtype) {
    if (R < 0 || gamma < 0 || V < 1) return SPEC_EINVAL;
    if (!dtype_ok(t_dtype) || !dtype_ok(d_dtype)) return SPEC_EDTYPE;
    if (gamma > kMaxGamma || V > SPEC_MAX_VERIFY_VOCAB) return SPEC_EUNSUPPORTED;
    Plan p;
    if (R > 0 && !make_plan(R, gamma + 1, V, p)) return SPEC_EUNSUPPORTED;
    const int ddt = gamma > 0 ? d_dtype : t_dtype;
    if (R == 0 || V % 8 != 0 || t_dtype != SPEC_BF16 || ddt != SPEC_BF16)
        return SPEC_PATH_SPLIT;
    VerifyArgs a{};
    a.R = R;
    a.gamma = gamma;
    a.V = V;
    a.UG = gamma + 1;
    a.C = p.C;
    int kl = 0;
    size_t lds = 0;
    long G = 0;
    return hold_applies(a, &kl, &lds, &G) ? SPEC_PATH_HELD : SPEC_PATH_SPLIT;
}

int spec_tv_accept_rate(const void *draft_logits, const void *target_logits, int dtype,
                        const float *temperature, int N, int V, float *out_cstar,
                        float *out_resid_mass, void *workspace, size_t workspace_bytes,
                        void *stream) {
    if (N < 0 || V < 1) return SPEC_EINVAL;
    if (!dtype_ok(dtype)) return SPEC_EDTYPE;
    if (V > SPEC_MAX_VERIFY_VOCAB) return SPEC_EUNSUPPORTED;
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
    return launch(a, dtype, dtype, p.N, vec, (hipStream_t)stream);
}

}  // extern "C"
