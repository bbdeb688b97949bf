// verify.hip -- batched lossless speculative-sampling verification and the
// analytic acceptance rate on gfx950: four stream-ordered launches per call.
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
// unit.  The three launches, in stream order:
//  1. stats_kernel: persistent wave64s stream every needed row exactly once
//     from HBM with 16-byte loads, the items balanced over the waves through a
//     per-block unit table in LDS.  Per item it writes the chunk's scaled max
//     mu and weight sum S = sum 2^(z s - mu) per row (s = log2(e) / T), or the
//     chunk argmax at T = 0.  Malformed requests get their outputs here.
//  2. tv_kernel: first, wave w folds units w, w + W, ... at T > 0 into their
//     row normalisers (M = max mu, Z = sum S 2^(mu - M)); then the pair items
//     at T > 0 again -- launch 1 has just streamed them, so they come from
//     the 256 MB Infinity Cache when they fit -- with each chunk's weights
//     rebuilt exactly as launch 1 made them; per item the chunk's
//     sum min(p, q) and residual mass.  An item whose unit is still being
//     folded waits for its normalisers.
//  3. tv_combine_kernel: one wave per unit.  At T > 0 a position runs its
//     accept test on the two gathered logits, sums c* and Res and, if
//     rejected, makes the residual draw; the bonus unit makes the
//     inverse-CDF draw from q.  At T = 0 the unit's argmax test settles it.
// Each unit's last step arrives on its request's counter; the wave completing
// a request applies prefix survival to the units' accept bits and writes the
// outputs, and returns the counter to zero.
// Words passed between waves are 64-bit (launch tag, payload) pairs written
// and read with agent-scope atomics, so a reader never mistakes a stale word
// (an earlier call's) for a current one.  The tag is kept on the device, so
// that a captured graph gets a new one at every replay: launch 1 reads the
// workspace's next tag and copies it to the call's slot, launches 2 and 3
// read that slot, and launch 3 stores the tag after it as the next (nothing
// of the call reads the next-tag slot after launch 1).  A wave only waits for
// words whose writers cannot be waiting on it: the statistics words of an
// earlier launch, the normalisers of launch 2's folds (which read only launch
// 1's words and run before their waves take any item, on a grid that never
// exceeds the kernel's resident capacity), and the records of the waves
// whose counter arrivals made it the request's last.  Every wait is bounded
// and raises SPEC_DEV_SPIN_TIMEOUT rather than spin forever.
#include <math.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

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

// Division of n < 2^31 by a fixed d (1 <= d <= 1024) by a multiply-high and
// a shift: m = floor(2^(31 + l) / d) + 1 with l = ceil(log2 d) (the
// round-up method for 31-bit dividends).
struct FastDiv {
    uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    f.l = 0;
    while ((1u << f.l) < d) ++f.l;
    f.m = d == 1 ? 0u : (uint32_t)((1ull << (31 + f.l)) / d + 1);
    return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    return f.d == 1 ? n : __umulhi(n, f.m) >> (f.l - 1);
}

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
    uint64_t *part;          // [units * C][4] single pass: per-tile partial normalisers
    uint64_t *dump;          // single pass: per-wave sink of discarded stores
    FastDiv divC, divCh;     // single pass: division by C and by ceil(C / 2)
    uint32_t *tvbase;        // [R] single pass: TV positions of the requests before r
    int single;              // the call takes the single pass
    int spS;                 // single pass: stream waves per workgroup (items per tile)
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

// Every lane with `act` reads the word at p until it carries `tag`, then
// returns its payload (0 for inactive lanes).  Called by every active lane of
// the wave.  The wait is bounded: past kSpinLimit polls, or once any wave of
// the launch has timed out, it raises SPEC_DEV_SPIN_TIMEOUT and returns.
__device__ __forceinline__ uint32_t await_lane(const uint64_t *p, bool act, uint32_t tag,
                                               Control *ctl) {
    uint64_t v = act ? ld_word(p) : 0;
    bool stale = act && (uint32_t)(v >> 32) != tag;
    uint32_t it = 0;
    while (__ballot(stale)) {
        if ((++it & 255u) == 0u &&
            (it > kSpinLimit || (atomic_load_u32(&ctl->status) & SPEC_DEV_SPIN_TIMEOUT))) {
            if (stale) atomic_or_u32(&ctl->status, SPEC_DEV_SPIN_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
        if (stale) {
            v = ld_word(p);
            stale = (uint32_t)(v >> 32) != tag;
        }
    }
    return (uint32_t)v;
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
__device__ __forceinline__ bool is_tv(const Item &x) { return x.i < x.l && x.T != 0.0f; }

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
    uint32_t incl = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t n = __shfl_up(incl, o, 64);
        if (lane >= o) incl += n;
    }
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

    // As load(), except that a vector past the row end reads `pad` (16 bytes
    // of -inf logits) instead, so the words need no fix().
    __device__ __forceinline__ void load_padded(const T *row, long c0, int V, const T *pad) {
        const T *base = row + c0;
        const uint32_t lane = (uint32_t)lane_id();
        const long left = (long)V - c0;
        rem = kLanes * N;
#pragma unroll
        for (int j = 0; j < N / EPV; ++j) {
            const uint32_t e = (j * kLanes + lane) * EPV;
            load_vec((long)e < left ? base : pad, (long)e < left ? e : 0u, j);
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

// Scaling of a row pair's chunk weights for min(p, q): p_v = e_d alpha_d and
// q_v = e_t alpha_t are compared as min(e_t kt, e_d kd) in units of `unit`
// probability.  kt = 1 (unit alpha_t) unless the draft scale exceeds the
// target's by more than 2^100; then kd = 1 (unit alpha_d).  Both products stay
// finite because every e is at most 1 (up to one rounding).
struct PairScale {
    float kt, kd, unit;
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

// The pair scale of a chunk with scaled maxima mut, mud: alpha = 2^(mu - M) / Z
// per row and kd = alpha_d / alpha_t, formed from products only (the
// reciprocals are the rows').
__device__ __forceinline__ PairScale pair_scale(float mut, float mud, const RowNorm &t,
                                                const RowNorm &d) {
    PairScale ps;
    const float et = (mut > -kInf) ? __builtin_amdgcn_exp2f(mut - t.M) : 0.0f;
    const float ed = (mud > -kInf) ? __builtin_amdgcn_exp2f(mud - d.M) : 0.0f;
    const double at = (double)et * t.rZ, ad = (double)ed * d.rZ;
    if (!(at > 0.0)) {
        // q vanishes on the chunk: min(p, q) = 0 and no residual
        ps.kt = 0.0f;
        ps.kd = 1.0f;
        ps.unit = (float)ad;
        return ps;
    }
    const double k = (ed > 0.0f) ? (double)ed * (double)__builtin_amdgcn_exp2f(t.M - mut) *
                                       ((double)t.Z * d.rZ)
                                 : 0.0;
    if (k <= 0x1p100) {
        ps.kt = 1.0f;
        ps.kd = (float)k;
        ps.unit = (float)at;
    } else {
        ps.kt = (float)((double)et * (double)__builtin_amdgcn_exp2f(d.M - mud) *
                        ((double)d.Z * t.rZ));
        ps.kd = 1.0f;
        ps.unit = (float)ad;
    }
    return ps;
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
// do (bounded as in await_lane).  out[k] = payload (0 for inactive words).
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
        const double incl = wave_incl_scan(wc);
        const double excl = run + incl - wc;
        const uint64_t hit = __ballot(c < C && excl + wc > t);
        const uint64_t pos = __ballot(c < C && wc > 0.0);
        if (pos) clast = b * 64 + 63 - __builtin_clzll(pos);
        if (hit) {
            const int k = __builtin_ctzll(hit);
            *tin = __shfl(t - excl, k, 64);
            return b * 64 + k;
        }
        run += __shfl(incl, 63, 64);
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
        const double incl = wave_incl_scan(tot);
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
        run += __shfl(incl, 63, 64);
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

// Row normalisers of unit x at T > 0 from the statistics pass's chunk words:
// M = max mu and Z = sum S 2^(mu - M), per lane over its chunks in
// increasing order, then across the wave in a fixed order, so that every wave
// folding the same unit gets the same bits.  A bonus row gives (Md, Zd) =
// (0, 1).
__device__ __forceinline__ void unit_norms(const VerifyArgs &a, const Item &x, float &Mt, float &Zt,
                                        float &Md, float &Zd) {
    const bool pair = is_pair(x);
    OnlineZ ot, od;
    fold_unit_words(a, x, pair, [&](const uint32_t (&w)[4]) {
        ot.add(__uint_as_float(w[0]), __uint_as_float(w[1]));
        if (pair) od.add(__uint_as_float(w[2]), __uint_as_float(w[3]));
    });
    ot.reduce(Mt, Zt);
    Md = 0.0f;
    Zd = 1.0f;
    if (pair) od.reduce(Md, Zd);
}

// The accept test of draft position x (T > 0) once its row normalisers are
// known: accept <=> q(x) >= p(x) or u < q(x)/p(x) (DART note eq. (3)), in
// fp64 from the two gathered logits of the draft token x_{i+1}; publishes the
// unit's record (flags, log q(x)).  The uniform's range is checked by the
// combine.
// The accept test on the gathered logits zx (target), dx (draft) of the draft
// token: q(x) >= p(x) or u < q(x)/p(x), in fp64; *lqx = log q(x).
__device__ __forceinline__ bool accept_eval(float zx, float dx, float s, float Mt, float Zt,
                                            float Md, float Zd, float uacc, float *lqx) {
    const double lq2 = (double)zx * (double)s - (double)Mt;
    const double lp2 = (double)dx * (double)s - (double)Md;
    const double q = exp2(lq2) / (double)Zt;
    const double pp = exp2(lp2) / (double)Zd;
    *lqx = (float)(lq2 * kLn2 - log((double)Zt));
    return q >= pp || (double)uacc < q / pp;
}

template <typename TT, typename TD>
__device__ __forceinline__ void accept_record(const VerifyArgs &a, const Item &x, float Mt,
                                              float Zt, float Md, float Zd) {
    const int xtok = a.tokens[(size_t)x.r * a.gamma + x.i];
    const float uacc = a.ua[(size_t)x.r * a.gamma + x.i];
    const bool valid = norms_ok(Mt, Zt) && norms_ok(Md, Zd) && xtok >= 0 && xtok < a.V;
    bool acc = false;
    float lqx = __builtin_nanf("");
    if (valid) {
        const float zx = load_one(row_ptr<TT>(a.zt, x.r, a.tG, x.i, a.V), xtok);
        const float dx = load_one(row_ptr<TD>(a.zd, x.r, a.dG, x.i, a.V), xtok);
        acc = accept_eval(zx, dx, x.s, Mt, Zt, Md, Zd, uacc, &lqx);
    }
    publish_n(a.rec + (size_t)x.u * kRecWords, a.tag, 2,
              (valid ? kFlagValid : 0u) | (acc ? kFlagAccept : 0u), __float_as_uint(lqx), 0u, 0u);
}

// The fold launch's work for draft position x at T > 0: its row normalisers
// for the TV items and the combine, then the accept test.
template <typename TT, typename TD>
__device__ __forceinline__ void norm_fold(const VerifyArgs &a, const Item &x) {
    float Mt, Zt, Md, Zd;
    unit_norms(a, x, Mt, Zt, Md, Zd);
    publish_n(a.nrm + (size_t)x.u * 4, a.tag, 4, __float_as_uint(Mt), __float_as_uint(Zt),
              __float_as_uint(Md), __float_as_uint(Zd));
    if (!a.tv_mode) accept_record<TT, TD>(a, x, Mt, Zt, Md, Zd);
}

// ---------------------------------------------------------------------------
// normalisers from the single pass's per-tile partials
// ---------------------------------------------------------------------------

// Row normalisers of one TV unit, as the stream waves use them.
struct SpNorm {
    RowNorm t, d;
};

// Fold of one unit's partials, partial e in lane e (lanes with `in`), in the
// wave's fixed reduction order, so that every workgroup gets the same bits.
__device__ __forceinline__ SpNorm sp_fold_partials(bool in, const uint32_t (&v)[4]) {
    OnlineZ ot, od;
    if (in) {
        ot.add(__uint_as_float(v[0]), __uint_as_float(v[1]));
        od.add(__uint_as_float(v[2]), __uint_as_float(v[3]));
    }
    float Mt, Zt, Md, Zd;
    ot.reduce(Mt, Zt);
    od.reduce(Md, Zd);
    SpNorm n;
    n.t = row_norm(Mt, Zt);
    n.d = row_norm(Md, Zd);
    return n;
}

// First item of partial e of the TV unit whose first item is f: f itself, then
// the start of every later tile (S items) the unit touches.
__device__ __forceinline__ uint32_t sp_part_item(uint32_t f, uint32_t e, uint32_t S) {
    return e == 0 ? f : (f / S + e) * S;
}
// Number of partials of the TV unit whose first item is f (C items).
__device__ __forceinline__ uint32_t sp_nparts(uint32_t f, uint32_t C, uint32_t S) {
    return (f + C - 1u) / S - f / S + 1u;
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
// position's row normalisers and accept test, and the chunk of the residual
// draw [q - p]_+ should this row be the request's first rejection (DART note
// eq. (3)-(4)).  Four-launch path: normalisers and accept record from the
// fold launch.  Single pass: normalisers folded here from the per-tile
// partials (the same fold as the coordinator's, so the same bits), and the
// accept test on the gathered logits.
template <typename TT, typename TD>
__device__ __forceinline__ void tv_unit(const VerifyArgs &a, const Item &x, UnitSum *s) {
    const int lane = lane_id();
    const int C = a.C, G = a.gamma;
    float usm = 0.0f, uacc = 0.0f;
    int xtok = 0;
    if (!a.tv_mode) {
        usm = a.us[(size_t)x.r * (G + 1) + x.i];
        uacc = a.ua[(size_t)x.r * G + x.i];
        xtok = a.tokens[(size_t)x.r * G + x.i];
    }
    constexpr int K = 2 * kCB + 4;
    const uint64_t *p[K];
    bool act[K];
    uint32_t o[K];
#pragma unroll
    for (int b = 0; b < kCB; ++b)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = b * 64 + lane;
            p[b * 2 + q] = a.st2 + ((size_t)x.u * C + c) * 2 + q;
            act[b * 2 + q] = c < C;
        }
    uint32_t np = 0;
    if (a.single) {
        // partial e of the unit in lane e
        const uint32_t S = (uint32_t)a.spS;
        const uint32_t f = (a.tvbase[x.r] + (uint32_t)x.i) * (uint32_t)C;
        np = sp_nparts(f, (uint32_t)C, S);
        const uint32_t ke = sp_part_item(f, (uint32_t)lane < np ? (uint32_t)lane : 0u, S);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            p[2 * kCB + w] = a.part + (size_t)ke * 4 + w;
            act[2 * kCB + w] = (uint32_t)lane < np;
        }
    } else {
        // lanes 0..3: normalisers; 4, 5: the fold's record (flags, log q(x))
        p[2 * kCB] = (lane < 4) ? a.nrm + (size_t)x.u * 4 + lane
                                : a.rec + (size_t)x.u * kRecWords + (lane & 1);
        act[2 * kCB] = lane < 4 || (!a.tv_mode && lane < 6);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            p[2 * kCB + w] = p[2 * kCB];
            act[2 * kCB + w] = false;
        }
    }
    await_batch<K>(p, act, a.tag, a.ctl, o, true);
    float Mt, Zt, Md, Zd;
    if (a.single) {
        const uint32_t vw[4] = {o[2 * kCB], o[2 * kCB + 1], o[2 * kCB + 2], o[2 * kCB + 3]};
        const SpNorm n = sp_fold_partials((uint32_t)lane < np, vw);
        Mt = n.t.M;
        Zt = n.t.Z;
        Md = n.d.M;
        Zd = n.d.Z;
    } else {
        Mt = __uint_as_float(rl(o[2 * kCB], 0));
        Zt = __uint_as_float(rl(o[2 * kCB], 1));
        Md = __uint_as_float(rl(o[2 * kCB], 2));
        Zd = __uint_as_float(rl(o[2 * kCB], 3));
    }
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
    } else if (a.single) {
        valid = norms_ok(Mt, Zt) && norms_ok(Md, Zd) && xtok >= 0 && xtok < a.V &&
                uniform_ok(uacc) && uniform_ok(usm);
        lqx = __builtin_nanf("");
        if (valid) {
            const float zx = load_one(row_ptr<TT>(a.zt, x.r, a.tG, x.i, a.V), xtok);
            const float dx = load_one(row_ptr<TD>(a.zd, x.r, a.dG, x.i, a.V), xtok);
            acc = accept_eval(zx, dx, x.s, Mt, Zt, Md, Zd, uacc, &lqx);
        }
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
    }
}

// T > 0 bonus unit (target row l_r): the row normalisers folded from the
// statistics words (as unit_norms folds them), and the chunk of the
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
        const float reft = exp_ref(mut), refd = exp_ref(mud);
        const double te = (ps.unit > 0.0f) ? su.tin / (double)ps.unit : INFINITY;
        float wv[N / EPV][EPV];
#pragma unroll
        for (int jj = 0; jj < N / EPV; ++jj)
#pragma unroll
            for (int q = 0; q < EPV; ++q) {
                const float et = ew(zt[jj][q], s, reft) * ps.kt;
                const float mn = __builtin_elementwise_minimum(et, ew(zd[jj][q], s, refd) * ps.kd);
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
    *lqd = (float)(((double)ztok * (double)s - (double)Mt) * kLn2 - log((double)Zt));
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
    else tv_unit<TT, TD>(a, x, s);
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
        else if (i < l) tv_unit<TT, TD>(a, x, &sum[i]);
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
    for (int k = lane; k <= G; k += 64) {
        const int32_t t = (k < A) ? a.tokens[(size_t)r * G + k] : (k == A ? tok : -1);
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
    publish_n(a.st1 + ((size_t)x.u * a.C + x.c) * 4, a.tag, 4, w0, w1, w2, w3);
}

// Item of unit u with chunk 0 (for the per-unit kernels); false if the unit
// is not active (request malformed, or i > l_r).
__device__ __forceinline__ bool unit_item(const VerifyArgs &a, long u, Item &x) {
    if (u >= (long)a.R * a.UG) return false;
    x.u = (int)u;
    x.r = (int)(u / a.UG);
    x.i = (int)(u % a.UG);
    x.c = 0;
    if (!request_ok(a, x.r, x.T, x.l) || x.i > x.l) return false;
    x.s = x.T != 0.0f ? exp2_scale(x.T) : 0.0f;
    return true;
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
// mu_d) and the row normalisers, the weights e = 2^(z s - mu) are rebuilt
// exactly as the statistics made them; *cmin = the chunk's sum min(p, q) and
// *cres its residual mass sum [q - p]_+.  The logits must be fixed (past-the-
// row slots -inf).
template <int N, typename RT, typename RD>
__device__ __forceinline__ void tv_sums(const RT &rt, const RD &rd, float s, float mut, float St,
                                        float mud, const RowNorm &nt, const RowNorm &nd,
                                        double *cmin, double *cres) {
    const PairScale ps = pair_scale(mut, mud, nt, nd);
    const float reft = exp_ref(mut), refd = exp_ref(mud);
    // min(p, q) in units of ps.unit, summed in the same slot order as the
    // chunk's weight sum in the statistics pass, so a chunk with q <= p
    // everywhere has a residual of exactly 0
    float acc = 0.0f, ssum;
    if (ps.kt == 1.0f) {
#pragma unroll
        for (int k = 0; k < N; ++k)
            acc += __builtin_elementwise_minimum(ew(rt.get(k), s, reft),
                                                 ew(rd.get(k), s, refd) * ps.kd);
        ssum = St;
    } else {
        float et[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
            et[k] = ew(rt.get(k), s, reft) * ps.kt;
            acc += __builtin_elementwise_minimum(et[k], ew(rd.get(k), s, refd));
        }
        ssum = wave_sum_f(lane_sum<N>(et));
    }
    const float smin = wave_sum_f(acc);
    *cmin = (double)ps.unit * (double)smin;
    *cres = fmax((double)ps.unit * ((double)ssum - (double)smin), 0.0);
}

// The same TV sums from the chunk's weights e_t, e_d as the statistics made
// them (so the same bits as tv_sums on the logits).
template <int N>
__device__ __forceinline__ void tv_sums_w(const float (&et)[N], const float (&ed)[N], float mut,
                                          float St, float mud, const RowNorm &nt,
                                          const RowNorm &nd, double *cmin, double *cres) {
    const PairScale ps = pair_scale(mut, mud, nt, nd);
    float acc = 0.0f, ssum;
    if (ps.kt == 1.0f) {
#pragma unroll
        for (int k = 0; k < N; ++k) acc += __builtin_elementwise_minimum(et[k], ed[k] * ps.kd);
        ssum = St;
    } else {
        float ek[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
            ek[k] = et[k] * ps.kt;
            acc += __builtin_elementwise_minimum(ek[k], ed[k]);
        }
        ssum = wave_sum_f(lane_sum<N>(ek));
    }
    const float smin = wave_sum_f(acc);
    *cmin = (double)ps.unit * (double)smin;
    *cres = fmax((double)ps.unit * ((double)ssum - (double)smin), 0.0);
}

// TV of pair item x at T > 0 (chunk re-read, from the Infinity Cache when the
// rows fit there), with the chunk's words and the unit's normalisers from the
// earlier launches (w8: lanes 0..3 the chunk's words, 4..7 the normalisers).
template <int N, typename RT, typename RD>
__device__ __forceinline__ void tv_item(const VerifyArgs &a, const Item &x, RT &rt, RD &rd,
                                        uint32_t w8) {
    rt.fix();
    rd.fix();
    double cmin, cres;
    const RowNorm nt = row_norm(__uint_as_float(rl(w8, 4)), __uint_as_float(rl(w8, 5)));
    const RowNorm nd = row_norm(__uint_as_float(rl(w8, 6)), __uint_as_float(rl(w8, 7)));
    tv_sums<N>(rt, rd, x.s, __uint_as_float(rl(w8, 0)), __uint_as_float(rl(w8, 1)),
               __uint_as_float(rl(w8, 2)), nt, nd, &cmin, &cres);
    publish_n(a.st2 + ((size_t)x.u * a.C + x.c) * 2, a.tag, 2, __float_as_uint((float)cmin),
              __float_as_uint((float)cres), 0u, 0u);
}

// Issues the loads of pair item x: its chunk of both rows, and (lanes 0..7)
// the chunk's words and the unit's normalisers.
template <typename TT, typename TD, int N, int EPV>
__device__ __forceinline__ uint64_t load_tv_item(const VerifyArgs &a, const Item &x,
                                                 RawChunk<TT, N, EPV> &rt,
                                                 RawChunk<TD, N, EPV> &rd) {
    const int lane = lane_id();
    const uint64_t *p = (lane < 4) ? a.st1 + ((size_t)x.u * a.C + x.c) * 4 + lane
                                   : a.nrm + (size_t)x.u * 4 + (lane & 3);
    // plain loads: both kinds of word were written by earlier launches
    const uint64_t w = (lane < 8) ? *p : 0;
    load_item(a, x, rt, rd);
    return w;
}

// Kernel 2: one wave per draft position at T > 0 folds launch 1's chunk
// words into the position's row normalisers and runs the accept test.
template <typename TT, typename TD, int N, int EPV>
__global__ void __launch_bounds__(kBlock) fold_kernel(VerifyArgs a) {
    a.tag = call_tag(a.ctl);
    Item y;
    if (unit_item(a, wave_index(), y) && y.T != 0.0f && is_pair(y)) norm_fold<TT, TD>(a, y);
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
        // lanes 0..3: launch 1's chunk words, 4..7: launch 2's normalisers
        if (__ballot(lane < 8 && (uint32_t)(w >> 32) != a.tag) && lane == 0)
            atomic_or_u32(&a.ctl->status, SPEC_DEV_SPIN_TIMEOUT);
        tv_item<N>(a, x, rt, rd, (uint32_t)w);
    }
}

// ===========================================================================
// single-pass path (target and draft logits of one dtype)
// ===========================================================================
//
// One persistent kernel streams every needed row once.  An item is two row
// chunks ("halves") of 64 kSpN logits:
//   * a TV item: chunk c of the target and of the draft row of a draft
//     position at T > 0 (these come first, position by position);
//   * a T = 0 position's target and draft chunk c;
//   * chunks 2m and 2m + 1 of a target row l_r (the bonus row).
// Item k goes to stream wave k mod S of workgroup (k / S) mod G in round
// k / (S G), so a workgroup's S items of one round are consecutive: a tile.
// Every workgroup has S stream waves and one coordinator wave.
//
// A stream wave keeps its loads kSpAhead rounds ahead in a register ring.  In
// round j it publishes the chunk words of its item (as the statistics launch
// does), hands them to the coordinator in LDS and keeps a TV item's logits in
// LDS; kSpLag rounds later, with the unit's row normalisers from the
// coordinator, it publishes the TV sums of the held chunks.
//
// The coordinator folds, once a tile's statistics are in, each TV unit's run
// of chunks in the tile into a partial (M, Z per row), lane by lane in item
// order, and publishes it at the run's first item.  One round later it
// gathers every partial of each TV unit of that tile (one per tile the unit
// touches), folds them in item order into the unit's normalisers and hands
// them to the stream waves; the workgroup holding the unit's first item also
// publishes them and runs the accept test.  A partial still missing after a
// bounded wait (its workgroup not resident) is made by the coordinator itself
// from the logits with the same arithmetic, so no workgroup depends on
// another being scheduled, and every fold of a unit gives the same bits.

constexpr int kSpN = 16;         // logits per lane of a row chunk (chunk = 1024 logits)
constexpr int kSpLag = 2;        // rounds from an item's statistics to its TV sums
constexpr int kSpMaxUnits = 2048;            // unit table entries (LDS)
constexpr uint32_t kSpHelpPolls = 64;        // polls of a missing partial before making it

// Per element type: kS stream waves per workgroup and kAhead rounds of loads
// in flight per wave, about 128 KB per compute unit.  A held TV item is its
// fp32 chunk weights (8 KB).  bf16: 7 + 1 waves, two per SIMD (256 registers
// each), two rounds of held items in 112 KB of LDS; fp32: 6 + 1 waves, 96 KB.
template <typename T> struct SpCfg;
template <> struct SpCfg<uint16_t> {
    static constexpr int kS = 7, kAhead = 4;
};
template <> struct SpCfg<float> {
    static constexpr int kS = 6, kAhead = 3;
};

enum : int { kSpTV = 0, kSpGreedy = 1, kSpRow = 2, kSpNone = 3 };

// 16 bytes of -inf logits per element type: the single pass loads them for the
// slots of a chunk past the row end.
__device__ uint32_t kNegInfBf16[4] = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
__device__ uint32_t kNegInfF32[4] = {0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
template <typename T> __device__ __forceinline__ const T *neg_inf_pad();
template <> __device__ __forceinline__ const uint16_t *neg_inf_pad<uint16_t>() {
    return reinterpret_cast<const uint16_t *>(kNegInfBf16);
}
template <> __device__ __forceinline__ const float *neg_inf_pad<float>() {
    return reinterpret_cast<const float *>(kNegInfF32);
}

// Item counts of the single pass (the same in every workgroup).
struct SpGrid {
    uint32_t n_tv, n_gr, n_row;   // units per group (TV positions, T = 0 positions, rows)
    uint32_t i_tv, i_gr, items;   // item boundaries of the groups
    uint32_t ch;                  // items per row unit: ceil(C / 2)
    uint32_t rounds;
};

struct SpItem {
    int kind, u, r, i, c0, c1;    // c1 < 0: the second half is unused
    float T, s;
};

// Unit table in LDS: TV positions, then T = 0 positions, then target rows l_r,
// each entry r << 8 | i, with the request's exp2 scale log2(e)/T (0 at T = 0)
// in tab_s (built by every workgroup from the request arrays), so that the
// streaming loop reads no request data from global memory.
__device__ __forceinline__ SpGrid sp_build_table(const VerifyArgs &a, uint32_t *tab,
                                                 float *tab_s, uint32_t (*scr)[16]) {
    const int nt = blockDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = nt >> 6;
    const int K = (a.R + nt - 1) / nt;
    const int r0 = tid * K, r1 = min(r0 + K, a.R);
    uint32_t c[3] = {0u, 0u, 0u};
    for (int r = r0; r < r1; ++r) {
        float T;
        int l;
        if (!request_ok(a, r, T, l)) continue;
        if (T != 0.0f) c[0] += (uint32_t)l;
        else c[1] += (uint32_t)l;
        if (!a.tv_mode) c[2] += 1u;
    }
    uint32_t incl[3], base[3], tot[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        incl[q] = c[q];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t n = __shfl_up(incl[q], o, 64);
            if (lane >= o) incl[q] += n;
        }
        if (lane == 63) scr[q][wave] = incl[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        base[q] = 0u;
        tot[q] = 0u;
        for (int w = 0; w < nw; ++w) {
            if (w < wave) base[q] += scr[q][w];
            tot[q] += scr[q][w];
        }
        base[q] += incl[q] - c[q];
    }
    if (blockIdx.x == 0) {
        // TV positions of the requests before r, for the combine launch
        uint32_t tb = base[0];
        for (int r = r0; r < r1; ++r) {
            float T;
            int l;
            a.tvbase[r] = tb;
            if (request_ok(a, r, T, l) && T != 0.0f) tb += (uint32_t)l;
        }
    }
    for (int r = r0; r < r1; ++r) {
        float T;
        int l;
        if (!request_ok(a, r, T, l)) continue;
        const uint32_t e = (uint32_t)r << 8;
        const float s = T != 0.0f ? exp2_scale(T) : 0.0f;
        if (T != 0.0f) {
            for (int i = 0; i < l; ++i) {
                tab_s[base[0]] = s;
                tab[base[0]++] = e | (uint32_t)i;
            }
        } else {
            for (int i = 0; i < l; ++i) {
                tab_s[tot[0] + base[1]] = s;
                tab[tot[0] + base[1]++] = e | (uint32_t)i;
            }
        }
        if (!a.tv_mode) {
            tab_s[tot[0] + tot[1] + base[2]] = s;
            tab[tot[0] + tot[1] + base[2]++] = e | (uint32_t)l;
        }
    }
    SpGrid g;
    g.n_tv = tot[0];
    g.n_gr = tot[1];
    g.n_row = tot[2];
    g.ch = ((uint32_t)a.C + 1u) / 2u;
    g.i_tv = g.n_tv * (uint32_t)a.C;
    g.i_gr = g.i_tv + g.n_gr * (uint32_t)a.C;
    g.items = g.i_gr + g.n_row * g.ch;
    return g;
}

// Item k (any k >= 0; past the end an unused item).  x.T is 0 at T = 0 and 1
// otherwise (the statistics only ask whether T is 0); x.s = log2(e)/T.
__device__ __forceinline__ SpItem sp_item(const VerifyArgs &a, const SpGrid &g,
                                          const uint32_t *tab, const float *tab_s, uint32_t k) {
    SpItem x;
    const uint32_t C = (uint32_t)a.C;
    uint32_t q = 0u;
    if (k < g.i_tv) {
        q = fdiv(k, a.divC);
        x.kind = kSpTV;
        x.c0 = x.c1 = (int)(k - q * C);
    } else if (k < g.i_gr) {
        const uint32_t k2 = k - g.i_tv, q2 = fdiv(k2, a.divC);
        x.kind = kSpGreedy;
        x.c0 = x.c1 = (int)(k2 - q2 * C);
        q = g.n_tv + q2;
    } else if (k < g.items) {
        const uint32_t k2 = k - g.i_gr, q2 = fdiv(k2, a.divCh), m = k2 - q2 * g.ch;
        x.kind = kSpRow;
        x.c0 = (int)(2u * m);
        x.c1 = (2u * m + 1u < C) ? (int)(2u * m + 1u) : -1;
        q = g.n_tv + g.n_gr + q2;
    } else {
        x.kind = kSpNone;
        x.c0 = 0;
        x.c1 = -1;
    }
    const uint32_t e = __builtin_amdgcn_readfirstlane(x.kind == kSpNone ? 0u : tab[q]);
    x.s = __uint_as_float(
        __builtin_amdgcn_readfirstlane(x.kind == kSpNone ? 0u : __float_as_uint(tab_s[q])));
    x.T = x.s != 0.0f ? 1.0f : 0.0f;
    x.r = (int)(e >> 8);
    x.i = (int)(e & 255u);
    x.u = x.r * a.UG + x.i;
    return x;
}

// Issues item x's loads (no branch: the slots past the row end and an unused
// half read the -inf pad).
template <typename T, int EPV>
__device__ __forceinline__ void sp_issue(const VerifyArgs &a, const SpItem &x,
                                         RawChunk<T, kSpN, EPV> &h0, RawChunk<T, kSpN, EPV> &h1) {
    const bool none = x.kind == kSpNone;
    const T *t0 = row_ptr<T>(a.zt, x.r, a.tG, x.i, a.V);
    const T *t1 = (x.kind == kSpRow) ? t0 : row_ptr<T>(a.zd, x.r, a.dG, x.i, a.V);
    const bool u1 = none || x.c1 < 0;
    const T *pad = neg_inf_pad<T>();
    h0.load_padded(none ? pad : t0, none ? 0 : (long)x.c0 * kLanes * kSpN, none ? 0 : a.V, pad);
    h1.load_padded(u1 ? pad : t1, u1 ? 0 : (long)x.c1 * kLanes * kSpN, u1 ? 0 : a.V, pad);
}

// Chunk words of one half: (scaled max mu, weight sum S) at T > 0, or
// (max value, its lowest id; 0xffffffff after a NaN) at T = 0.
template <int N, int EPV, typename RC>
__device__ __forceinline__ void half_words(const RC &rc, float T, float s, long c0, uint32_t &w0,
                                           uint32_t &w1, float (&e)[N]) {
    if (T == 0.0f) {
        float bv;
        int bi, bad;
        chunk_argmax<N, EPV>(rc, c0, bv, bi, bad);
        w0 = __float_as_uint(bv);
        w1 = bad ? 0xffffffffu : (uint32_t)bi;
#pragma unroll
        for (int k = 0; k < N; ++k) e[k] = 0.0f;
    } else {
        float mu, S;
        chunk_exp<N>(rc, s, e, mu, S);
        w0 = __float_as_uint(mu);
        w1 = __float_as_uint(S);
    }
}

// The four chunk words of item x (loaded by sp_issue): words 0, 1 of half 0,
// words 2, 3 of half 1, and (T > 0) the chunk weights of both halves.  Every
// wave computing them (stream or coordinator) runs this function, so they
// carry the same bits.
template <typename T, int EPV>
__device__ __forceinline__ void sp_item_words(const SpItem &x, RawChunk<T, kSpN, EPV> &h0,
                                              RawChunk<T, kSpN, EPV> &h1, uint32_t (&w)[4],
                                              float (&e0)[kSpN], float (&e1)[kSpN]) {
    half_words<kSpN, EPV>(h0, x.T, x.s, (long)x.c0 * kLanes * kSpN, w[0], w[1], e0);
    half_words<kSpN, EPV>(h1, x.T, x.s, (long)(x.c1 < 0 ? 0 : x.c1) * kLanes * kSpN, w[2], w[3],
                          e1);
}

// The sink of a discarded store of this wave.
__device__ __forceinline__ uint64_t *sp_dump(const VerifyArgs &a) {
    return a.dump + ((blockIdx.x & 255u) * 16u + (threadIdx.x >> 6)) * 4u;
}

// Lane q of the result holds w[q & 3] (w wave-uniform): two selects on the
// lane's bits, so that no lane indexes the array.
__device__ __forceinline__ uint32_t lanes4(const uint32_t (&w)[4]) {
    const int lane = lane_id();
    const uint32_t lo = (lane & 1) ? w[1] : w[0];
    const uint32_t hi = (lane & 1) ? w[3] : w[2];
    return (lane & 2) ? hi : lo;
}

// Publishes item x's chunk words (v: lane q holds word q): a position's four
// at its chunk, a row item's two per chunk.
__device__ __forceinline__ void sp_publish_words(const VerifyArgs &a, const SpItem &x,
                                                 uint32_t v) {
    const int lane = lane_id();
    const bool second = x.kind == kSpRow && lane >= 2;
    const int c = second ? x.c1 : x.c0;
    const int q = second ? lane - 2 : lane;
    const bool dumped = x.kind == kSpNone || (second && x.c1 < 0);
    uint64_t *p = dumped ? sp_dump(a) + (lane & 3) : a.st1 + ((size_t)x.u * a.C + c) * 4 + q;
    if (lane < 4) st_word(p, a.tag, v);
}

// Partial normalisers of the lanes in `in` (lane w holding the words of item
// tile * S + w): M = max mu, Z = sum S 2^(mu - M) per row, in the wave's fixed
// reduction order.
__device__ __forceinline__ void sp_fold_lanes(bool in, const uint32_t (&w)[4], float &Mt,
                                              float &Zt, float &Md, float &Zd) {
    OnlineZ ot, od;
    if (in) {
        ot.add(__uint_as_float(w[0]), __uint_as_float(w[1]));
        od.add(__uint_as_float(w[2]), __uint_as_float(w[3]));
    }
    ot.reduce(Mt, Zt);
    od.reduce(Md, Zd);
}

// The run of TV unit q's items in the tile holding item k0 (k0 the run's
// first item): [k0, end).
__device__ __forceinline__ uint32_t sp_run_end(const VerifyArgs &a, uint32_t q, uint32_t k0,
                                               int S) {
    const uint32_t tile_end = (k0 / (uint32_t)S + 1u) * (uint32_t)S;
    const uint32_t unit_end = (q + 1u) * (uint32_t)a.C;
    return tile_end < unit_end ? tile_end : unit_end;
}

// The coordinator's own statistics of TV unit q's run [k0, end), when the
// workgroup that streams it has not published it: the run's items are loaded
// and their words made exactly as a stream wave makes them, each in the lane
// of its place in the tile, and folded as the tile's coordinator folds them.
template <typename T, int EPV, int S>
__device__ __forceinline__ void sp_make_partial(const VerifyArgs &a, const SpGrid &g,
                                             const uint32_t *tab, const float *tab_s,
                                             uint32_t k0, uint32_t end, float (&P)[4]) {
    const int lane = lane_id();
    const uint32_t tile0 = k0 / (uint32_t)S * (uint32_t)S;
    uint32_t mine[4] = {0u, 0u, 0u, 0u};
    for (uint32_t k = k0; k < end; ++k) {
        const SpItem x = sp_item(a, g, tab, tab_s, k);
        RawChunk<T, kSpN, EPV> h0, h1;
        sp_issue<T, EPV>(a, x, h0, h1);
        uint32_t w[4];
        float e0[kSpN], e1[kSpN];
        sp_item_words<T, EPV>(x, h0, h1, w, e0, e1);
        if ((uint32_t)lane == k - tile0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) mine[q] = w[q];
        }
    }
    const bool in = (uint32_t)lane >= k0 - tile0 && (uint32_t)lane < end - tile0;
    sp_fold_lanes(in, mine, P[0], P[1], P[2], P[3]);
}

// Loads of a batch of partials (units q .. qe - 1 of a tile, at most 64
// partials, partial e of a unit in lane off_unit + e), issued ahead of their
// use.
struct SpFetch {
    uint64_t v[4];
    uint32_t ke;
    int ui;
    uint32_t q, qe;
};

template <int S>
__device__ __forceinline__ SpFetch sp_fetch_issue(const VerifyArgs &a, uint32_t q, uint32_t qb) {
    const int lane = lane_id();
    const uint32_t C = (uint32_t)a.C;
    SpFetch f;
    f.q = q;
    uint32_t qe = q, used = 0;
    // np <= 64 for C <= 256 and S >= 6
    while (qe <= qb && (qe == q || used + sp_nparts(qe * C, C, S) <= 64u))
        used += sp_nparts((qe++) * C, C, S);
    f.qe = qe;
    f.ke = 0;
    f.ui = -1;
    uint32_t off = 0;
    for (uint32_t u = q; u < qe; ++u) {
        const uint32_t np = sp_nparts(u * C, C, S);
        if ((uint32_t)lane >= off && (uint32_t)lane < off + np) {
            f.ui = (int)(u - q);
            f.ke = sp_part_item(u * C, (uint32_t)lane - off, (uint32_t)S);
        }
        off += np;
    }
    const bool act = f.ui >= 0;
    const uint64_t *pp = a.part + (size_t)f.ke * 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) f.v[w] = act ? ld_word(pp + w) : ((uint64_t)a.tag << 32);
    return f;
}

// Completes a batch: partials not current yet are polled; one still missing
// after a bounded wait (its workgroup not resident) is made here and
// published.  Each unit's partials are then moved to lanes 0.. and folded
// into out[u - qa].
template <typename T, int EPV, int S>
__device__ __forceinline__ void sp_fetch_finish(const VerifyArgs &a, const SpGrid &g,
                                                const uint32_t *tab, const float *tab_s,
                                                SpFetch &f, uint32_t qa, SpNorm *out) {
    const int lane = lane_id();
    const uint32_t C = (uint32_t)a.C;
    const bool act = f.ui >= 0;
    const uint64_t *pp = a.part + (size_t)f.ke * 4;
    for (uint32_t polls = 0;; ++polls) {
        bool stale = false;
#pragma unroll
        for (int w = 0; w < 4; ++w) stale = stale || (uint32_t)(f.v[w] >> 32) != a.tag;
        const uint64_t sm = __ballot(stale);
        if (!sm) break;
        if (polls >= kSpHelpPolls) {
            for (uint64_t m = sm; m; m &= m - 1) {
                const int e = __builtin_ctzll(m);
                const uint32_t k0 = rl(f.ke, e);
                const uint32_t u = f.q + (uint32_t)__builtin_amdgcn_readlane(f.ui, e);
                float P[4];
                sp_make_partial<T, EPV, S>(a, g, tab, tab_s, k0, sp_run_end(a, u, k0, S), P);
                publish_n(a.part + (size_t)k0 * 4, a.tag, 4, __float_as_uint(P[0]),
                          __float_as_uint(P[1]), __float_as_uint(P[2]), __float_as_uint(P[3]));
                if (lane == e) {
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        f.v[w] = ((uint64_t)a.tag << 32) | __float_as_uint(P[w]);
                }
            }
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (act && (uint32_t)(f.v[w] >> 32) != a.tag) f.v[w] = ld_word(pp + w);
    }
    uint32_t vw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) vw[w] = (uint32_t)f.v[w];
    uint32_t off = 0;
    for (uint32_t u = f.q; u < f.qe; ++u) {
        const uint32_t np = sp_nparts(u * C, C, S);
        uint32_t mv[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
            mv[w] = (uint32_t)__shfl((int)vw[w], (int)((uint32_t)lane + off) & 63, 64);
        const SpNorm n = sp_fold_partials((uint32_t)lane < np, mv);
        if (lane == 0) out[u - qa] = n;
        off += np;
    }
}

// LDS state of a single-pass workgroup.
template <typename T, int EPV, int S>
struct SpShared {
    static constexpr int kV4 = kSpN / 4;  // 16-byte words of a half's weights per lane
    uint4 hold[kSpLag][S][2][kV4][64];    // TV items' weights, per round slot and wave
    uint32_t cw[kSpLag + 1][S][4];       // chunk words of each wave's item
    SpNorm nrm[kSpLag][S];               // normalisers of the tile's TV units
    uint32_t done[S];                    // rounds whose statistics each wave has handed over
    uint32_t ready[kSpLag];              // round + 1 once the tile's normalisers are in
    uint32_t scr[3][16];
    uint32_t tab[kSpMaxUnits];
    float tab_s[kSpMaxUnits];
};

__device__ __forceinline__ uint32_t lds_load(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The coordinator wave (see above).  Round j: the loads of tile j - 1's
// partials are issued first; once the stream waves have handed over round j,
// tile j's partials are published; then tile j - 1's normalisers are folded
// and handed to the stream waves.
template <typename TT, typename TD, typename T, int EPV, int S>
__device__ __forceinline__ void sp_coordinator(const VerifyArgs &a, const SpGrid &g,
                                               SpShared<T, EPV, S> &sh) {
    const int lane = lane_id();
    const uint32_t C = (uint32_t)a.C, G = gridDim.x;
    for (uint32_t j = 0; j <= g.rounds; ++j) {
        // tile j - 1: its TV units qa..qb, first batch of partial loads
        const uint32_t jp = j - 1u;
        const uint32_t kp = (jp * G + blockIdx.x) * (uint32_t)S;
        const bool any = j >= 1 && kp < g.i_tv;
        const uint32_t qa = any ? fdiv(kp, a.divC) : 0u;
        const uint32_t qb = any ? fdiv(min(kp + (uint32_t)S, g.i_tv) - 1u, a.divC) : 0u;
        SpFetch f;
        if (any) f = sp_fetch_issue<S>(a, qa, qb);
        if (j < g.rounds) {
            uint32_t spins = 0;
            while (__ballot(lane < S && lds_load(&sh.done[lane < S ? lane : 0]) < j + 1u)) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > kSpinLimit) {
                    if (lane == 0) atomic_or_u32(&a.ctl->status, SPEC_DEV_SPIN_TIMEOUT);
                    break;
                }
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const uint32_t k0 = (j * G + blockIdx.x) * (uint32_t)S;
            if (k0 < g.i_tv) {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                const uint32_t k = k0 + (uint32_t)lane;
                const bool tv = lane < S && k < g.i_tv;
                if (lane < S) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[q] = sh.cw[j % (kSpLag + 1)][lane][q];
                }
                const uint32_t qk = fdiv(k, a.divC);
                const uint32_t kl = min(k0 + (uint32_t)S, g.i_tv) - 1u;
                for (uint32_t q = fdiv(k0, a.divC); q <= fdiv(kl, a.divC); ++q) {
                    float P[4];
                    sp_fold_lanes(tv && qk == q, w, P[0], P[1], P[2], P[3]);
                    const uint32_t kf = max(q * C, k0);
                    publish_n(a.part + (size_t)kf * 4, a.tag, 4, __float_as_uint(P[0]),
                              __float_as_uint(P[1]), __float_as_uint(P[2]),
                              __float_as_uint(P[3]));
                }
            }
        }
        if (j >= 1) {
            if (any) {
                SpNorm *out = sh.nrm[jp % kSpLag];
                sp_fetch_finish<T, EPV, S>(a, g, sh.tab, sh.tab_s, f, qa, out);
                for (uint32_t q = f.qe; q <= qb;) {
                    SpFetch f2 = sp_fetch_issue<S>(a, q, qb);
                    sp_fetch_finish<T, EPV, S>(a, g, sh.tab, sh.tab_s, f2, qa, out);
                    q = f2.qe;
                }
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (lane == 0) lds_store(&sh.ready[jp % kSpLag], jp + 1u);
        }
    }
}

// A stream wave (see above).  Iteration j: the loads of round j + kAhead,
// the statistics of round j, then the TV sums of round j - kSpLag from the
// weights held in LDS slot (j - kSpLag) % kSpLag, whose place round j's
// weights then take.
template <typename T, int EPV, int S>
__device__ __forceinline__ void sp_stream(const VerifyArgs &a, const SpGrid &g,
                                          SpShared<T, EPV, S> &sh, int wave) {
    using RC = RawChunk<T, kSpN, EPV>;
    constexpr int kV4 = SpShared<T, EPV, S>::kV4;
    constexpr int kSpAhead = SpCfg<T>::kAhead, kSpRing = kSpAhead + 1;
    const int lane = lane_id();
    const uint32_t C = (uint32_t)a.C;
    const uint32_t kb = blockIdx.x * (uint32_t)S + (uint32_t)wave;
    const uint32_t stride = gridDim.x * (uint32_t)S;
    auto item_of = [&](uint32_t j) -> uint32_t {
        // past the last round the item index may not fit 32 bits: clamp
        return j < g.rounds + kSpAhead + kSpLag ? kb + j * stride : 0xffffffffu;
    };
    RC h0[kSpRing], h1[kSpRing];
#pragma unroll
    for (int q = 0; q < kSpAhead; ++q)
        sp_issue<T, EPV>(a, sp_item(a, g, sh.tab, sh.tab_s, item_of((uint32_t)q)), h0[q], h1[q]);
    for (uint32_t j0 = 0;; j0 += kSpRing) {
#pragma unroll
        for (int t = 0; t < kSpRing; ++t) {
            const uint32_t j = j0 + (uint32_t)t;
            if (j >= g.rounds + kSpLag) return;
            const uint32_t hs = j % kSpLag;  // LDS slot of round j (and of round j - kSpLag)
            // loads of round j + kAhead
            {
                const int ns = (t + kSpAhead) % kSpRing;
                sp_issue<T, EPV>(a, sp_item(a, g, sh.tab, sh.tab_s, item_of(j + kSpAhead)),
                                 h0[ns], h1[ns]);
            }
            // statistics of round j (ring slot t): chunk words published and
            // handed to the coordinator; the weights stay in registers
            const int rs = t;
            float e0[kSpN], e1[kSpN];
            {
                const SpItem x = sp_item(a, g, sh.tab, sh.tab_s, item_of(j));
                uint32_t w[4];
                sp_item_words<T, EPV>(x, h0[rs], h1[rs], w, e0, e1);
                const uint32_t v = lanes4(w);
                sp_publish_words(a, x, v);
                if (lane < 4) sh.cw[j % (kSpLag + 1)][wave][lane] = v;
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                if (lane == 0) lds_store(&sh.done[wave], j + 1u);
            }
            // TV sums of round j - kSpLag, then round j's weights into its slot
            {
                const bool live = j >= (uint32_t)kSpLag;
                const uint32_t jt = live ? j - kSpLag : 0u;
                const uint32_t k = kb + jt * stride;
                const SpItem x = sp_item(a, g, sh.tab, sh.tab_s, live ? k : 0xffffffffu);
                if (live && jt < g.rounds) {
                    uint32_t spins = 0;
                    while (lds_load(&sh.ready[hs]) != jt + 1u) {
                        __builtin_amdgcn_s_sleep(1);
                        if (++spins > kSpinLimit) {
                            if (lane == 0) atomic_or_u32(&a.ctl->status, SPEC_DEV_SPIN_TIMEOUT);
                            break;
                        }
                    }
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                }
                float et[kSpN], ed[kSpN];
#pragma unroll
                for (int v = 0; v < kV4; ++v) {
                    const uint4 p0 = sh.hold[hs][wave][0][v][lane];
                    const uint4 p1 = sh.hold[hs][wave][1][v][lane];
                    et[v * 4 + 0] = __uint_as_float(p0.x); et[v * 4 + 1] = __uint_as_float(p0.y);
                    et[v * 4 + 2] = __uint_as_float(p0.z); et[v * 4 + 3] = __uint_as_float(p0.w);
                    ed[v * 4 + 0] = __uint_as_float(p1.x); ed[v * 4 + 1] = __uint_as_float(p1.y);
                    ed[v * 4 + 2] = __uint_as_float(p1.z); ed[v * 4 + 3] = __uint_as_float(p1.w);
                }
                const bool tv = x.kind == kSpTV;
                const uint32_t q = tv ? fdiv(k, a.divC) : 0u;
                const uint32_t q0 = tv ? fdiv(k - (uint32_t)wave, a.divC) : 0u;
                const SpNorm &nm = sh.nrm[hs][q - q0];
                const uint32_t *cw = sh.cw[jt % (kSpLag + 1)][wave];
                double cmin, cres;
                tv_sums_w<kSpN>(et, ed, __uint_as_float(cw[0]), __uint_as_float(cw[1]),
                                __uint_as_float(cw[2]), nm.t, nm.d, &cmin, &cres);
                uint64_t *p = tv ? a.st2 + ((size_t)x.u * C + x.c0) * 2 + (lane & 1)
                                 : sp_dump(a) + (lane & 1);
                const float cv = (float)cmin, rv = (float)cres;
                if (lane < 2) st_word(p, a.tag, __float_as_uint(lane == 0 ? cv : rv));
#pragma unroll
                for (int v = 0; v < kV4; ++v) {
                    sh.hold[hs][wave][0][v][lane] =
                        make_uint4(__float_as_uint(e0[v * 4]), __float_as_uint(e0[v * 4 + 1]),
                                   __float_as_uint(e0[v * 4 + 2]), __float_as_uint(e0[v * 4 + 3]));
                    sh.hold[hs][wave][1][v][lane] =
                        make_uint4(__float_as_uint(e1[v * 4]), __float_as_uint(e1[v * 4 + 1]),
                                   __float_as_uint(e1[v * 4 + 2]), __float_as_uint(e1[v * 4 + 3]));
                }
            }
        }
    }
}

// The single-pass kernel: S stream waves and one coordinator per workgroup,
// one workgroup per compute unit.
template <typename TT, typename TD, typename T, int EPV>
__global__ void __launch_bounds__((SpCfg<T>::kS + 1) * 64, 1) sp_kernel(VerifyArgs a) {
    constexpr int S = SpCfg<T>::kS;
    __shared__ SpShared<T, EPV, S> sh;
    a.tag = first_launch_tag(a.ctl);
    SpGrid g = sp_build_table(a, sh.tab, sh.tab_s, sh.scr);
    const uint32_t per_round = gridDim.x * (uint32_t)S;
    g.rounds = (g.items + per_round - 1u) / per_round;
    if (threadIdx.x < S) sh.done[threadIdx.x] = 0u;
    if (threadIdx.x < kSpLag) sh.ready[threadIdx.x] = 0u;
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (wave == S)
        sp_coordinator<TT, TD, T, EPV, S>(a, g, sh);
    else
        sp_stream<T, EPV, S>(a, g, sh, wave);
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
    size_t off_st1, off_st2, off_nrm, off_rec, off_part, off_dump, off_tvb, bytes;
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
    p.off_part = round_up(p.off_rec + 8 * kRecWords * (size_t)units, 256);
    p.off_dump = round_up(p.off_part + 32 * (size_t)units * C, 256);
    p.off_tvb = round_up(p.off_dump + 32 * 256 * 16, 256);
    p.bytes = round_up(p.off_tvb + 4 * (size_t)R, 256);
    return true;
}

size_t plan_bytes(long R, long upr, long V) {
    Plan p;
    return make_plan(R, upr, V, p) ? p.bytes : 0;
}

bool dtype_ok(int d) { return d == SPEC_F32 || d == SPEC_BF16; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Resident workgroups of a kernel with `lds` bytes of dynamic shared memory on
// the current device (cached per kernel, device and size).
long resident_blocks(const void *kernel, size_t lds) {
    struct Entry { const void *k; int dev; size_t lds; long cap; };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry &e : cache)
        if (e.k == kernel && e.dev == dev && e.lds == lds) return e.cap;
    int nb = 0, ncu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kBlock, lds) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const long cap = (long)nb * ncu;
    cache.push_back(Entry{kernel, dev, lds, cap});
    return cap;
}


// Compute units of the current device (cached per device; 0 if unknown).
long device_cus() {
    static std::mutex mu;
    static std::vector<std::pair<int, int>> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto &e : cache)
        if (e.first == dev) return e.second;
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    cache.emplace_back(dev, ncu);
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

// Shared memory of the unit table (0: too large, walk all candidates).
constexpr size_t kMaxTableBytes = 32768;
size_t table_bytes(const VerifyArgs &a) {
    const size_t b = 4 * (3 * (size_t)a.R + (size_t)a.R * a.UG);
    return b <= kMaxTableBytes ? (b + 255) / 256 * 256 : 0;
}

// Which path a call takes: the four-launch path, or with
// SPECVERIFY_PATH=single the single pass where it applies (one dtype for both
// tensors, 16-byte vector loads, a unit table that fits in LDS).  The tests
// run both.
bool single_pass_allowed() {
    const char *e = getenv("SPECVERIFY_PATH");
    return e && e[0] == 's';
}

template <typename TT, typename TD, int N, int EPV>
int launch_single(VerifyArgs a, hipStream_t st) {
    using T = TT;
    constexpr int S = SpCfg<T>::kS;
    const long cus = device_cus();
    const long grid = cus > 0 ? cus : 256;
    const long gc = a.tv_mode ? (a.R + kReqWaves - 1) / kReqWaves : a.R;
    a.tag = 0;  // read on the device by every launch
    a.single = 1;
    a.spS = S;
    hipLaunchKernelGGL((sp_kernel<TT, TD, T, EPV>), dim3((unsigned)grid), dim3((S + 1) * 64), 0,
                       st, a);
    hipLaunchKernelGGL((combine_kernel<TT, TD, N, EPV>), dim3((unsigned)gc), dim3(kReqBlock), 0,
                       st, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

template <typename TT, typename TD, int N, int EPV>
int launch_kernels(VerifyArgs a, hipStream_t st) {
    if constexpr (std::is_same<TT, TD>::value && N == kSpN && EPV == ChunkGeom<TT, TD, N>::kVec &&
                  EPV > 1) {
        if (single_pass_allowed() && (long)a.R * a.UG <= kSpMaxUnits)
            return launch_single<TT, TD, N, EPV>(a, st);
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
    hipLaunchKernelGGL((stats_kernel<TT, TD, N, EPV>), dim3((unsigned)g1), dim3(kBlock), lds, st,
                       a);
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
    a.part = (uint64_t *)(b + p.off_part);
    a.dump = (uint64_t *)(b + p.off_dump);
    a.tvbase = (uint32_t *)(b + p.off_tvb);
    a.C = p.C;
}

}  // namespace
}  // namespace sv

using namespace sv;

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
    a.divC = make_fastdiv((uint32_t)p.C);
    a.divCh = make_fastdiv((uint32_t)(p.C + 1) / 2);
    const bool vec = (V % 8 == 0) && aligned16(target_logits) &&
                     (gamma == 0 || aligned16(draft_logits));
    // with gamma == 0 no draft row exists; the draft type only shapes the plan
    const int ddt = gamma > 0 ? d_dtype : t_dtype;
    return launch(a, t_dtype, ddt, p.N, vec, (hipStream_t)stream);
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
    a.divC = make_fastdiv((uint32_t)p.C);
    a.divCh = make_fastdiv((uint32_t)(p.C + 1) / 2);
    const bool vec = (V % 8 == 0) && aligned16(target_logits) && aligned16(draft_logits);
    return launch(a, dtype, dtype, p.N, vec, (hipStream_t)stream);
}

}  // extern "C"
