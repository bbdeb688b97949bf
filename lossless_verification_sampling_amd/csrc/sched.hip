// sched.hip -- confidence-scheduled verify lengths on gfx950.
//
// Method (DSpark paper guide, personal-site-bgy.pages.dev, "scheduler"): the
// survival probability of draft position j of request r is the running product
// a[r][j] = c[r][1] ... c[r][j] of the confidence head's outputs.  A verify step
// of lengths l_r sends B = sum_r (1 + l_r) rows to the target and expects
// tau = sum_r (1 + sum_{j <= l_r} a[r][j]) accepted tokens, at SPS(B) steps per
// second (a profiled table), so the throughput is Theta = tau SPS(B).  Every
// candidate (r, j) enters one pool in descending a; candidates are admitted
// from the top and the walk stops at the first admission that does not raise
// Theta (the early stop that keeps the choice causal).  The asynchronous
// production variant admits the top K of the same order instead.
//
// One workgroup of 1024 threads:
//  1. the confidences come into LDS with coalesced loads (with the table
//     entries each thread needs later); each thread forms the fp32 products
//     of its requests left to right and writes 64-bit keys (inverted float bits of a, then r gamma + j - 1), so
//     an ascending sort gives a descending, ties by request then position --
//     the order that keeps every request's admissions a prefix;
//  2. bitonic sort of the keys (in registers with lane shuffles up to 1024
//     candidates, in LDS beyond);
//  3. each thread takes a run of consecutive sorted candidates: fp64 prefix
//     sums of a (thread runs, then a block scan) give tau after each
//     admission, Theta follows from the table, and a block minimum finds the
//     first candidate whose admission fails (Theta not raised, or B past the
//     table);
//  4. the admitted candidates raise their request's length with LDS atomics.
#include <math.h>

#include "common.h"

namespace sv {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kSchedMaxPool = SPEC_SCHED_MAX_POOL;
constexpr int kSchedPer = kSchedMaxPool / kSchedThreads;  // sorted candidates per thread at most

struct SchedArgs {
    const float *conf;  // [R][gamma]
    const float *sps;   // [bmax + 1]
    int R, gamma, bmax, topk;
    int P;              // power of two >= R gamma (at least 1)
    int32_t *out_len;   // [R]
    double *out_theta;  // [1] or null
    Control *ctl;
};

__global__ void __launch_bounds__(kSchedThreads) sched_kernel(SchedArgs a) {
    __shared__ uint64_t key[kSchedMaxPool];
    __shared__ int len[kSchedMaxPool];
    __shared__ float cf[kSchedMaxPool];
    __shared__ double wsum[kSchedWaves];
    __shared__ double last_theta[kSchedThreads];
    __shared__ int first_stop;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = a.R, G = a.gamma, N = R * G, P = a.P;
    // thread t later takes the sorted candidates [t E, (t + 1) E)
    const int E = P > kSchedThreads ? P / kSchedThreads : 1;
    const int k0 = tid * E;

    // ---- 1. every global load at once: confidences (to LDS), the table
    // entries this thread's candidates will need, validation ----------------
    int bad = 0;
    for (int k = tid; k < N; k += kSchedThreads) {
        const float c = a.conf[k];
        if (!(c >= 0.0f && c <= 1.0f)) bad = 1;
        cf[k] = c;
    }
    for (int b = tid; b <= a.bmax; b += kSchedThreads) {
        const float v = a.sps[b];
        if (!(v >= 0.0f && v <= 3.402823466e38f)) bad = 1;
    }
    float tab[kSchedPer];
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e) {
        const long B = (long)R + k0 + e + 1;  // batch after admitting candidates 0..k0+e
        tab[e] = (e < E && B <= a.bmax) ? a.sps[B] : 0.0f;
    }
    const float tab0 = R <= a.bmax ? a.sps[R] : 0.0f;
    __syncthreads();
    for (int r = tid; r < R; r += kSchedThreads) {
        float run = 1.0f;
        for (int j = 0; j < G; ++j) {
            run = run * cf[r * G + j];
            // +0.0 for -0.0, so that the float bits order the value
            const uint32_t bits = __float_as_uint(run + 0.0f);
            key[r * G + j] = ((uint64_t)(~bits) << 32) | (uint32_t)(r * G + j);
        }
        len[r] = 0;
    }
    for (int k = N + tid; k < P; k += kSchedThreads) key[k] = ~0ull;
    bad = __syncthreads_or(bad);
    if (bad) {
        for (int r = tid; r < R; r += kSchedThreads) a.out_len[r] = -1;
        if (tid == 0) {
            if (a.out_theta) a.out_theta[0] = __builtin_nan("");
            atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
        }
        return;
    }

    // ---- 2. bitonic sort, ascending keys ----------------------------------
    if (P <= kSchedThreads) {
        // one key per thread in registers: partners in the same wave come by
        // lane shuffle, partners 64 or more apart through LDS
        uint64_t v = tid < P ? key[tid] : ~0ull;
        for (int k = 2; k <= P; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                uint64_t w;
                if (j >= 64) {
                    __syncthreads();
                    key[tid] = v;
                    __syncthreads();
                    w = key[tid ^ j];
                } else {
                    w = __shfl_xor(v, j, 64);
                }
                const bool lower = (tid & j) == 0, up = (tid & k) == 0;
                v = (lower == up) ? (v < w ? v : w) : (v < w ? w : v);
            }
        }
        __syncthreads();
        if (tid < P) key[tid] = v;
        __syncthreads();
    } else {
        // several keys per thread: the same network in LDS.  A stage with
        // j < 64 pairs elements of one aligned run of 64, which the lanes of
        // one wave own (element i belongs to thread i mod 1024); a wave's LDS
        // accesses complete in order, so such stages need no block barrier.
        for (int k = 2; k <= P; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < P; i += kSchedThreads) {
                    const int l = i ^ j;
                    if (l > i) {
                        const uint64_t x = key[i], y = key[l];
                        const bool up = (i & k) == 0;
                        if ((x > y) == up) {
                            key[i] = y;
                            key[l] = x;
                        }
                    }
                }
                // a block barrier before any stage that reads across waves:
                // after a cross-wave stage, and after the last stage of a
                // phase that the next phase (first stage j = k) or the scan
                // reads across waves
                if (j >= 64 || (j == 1 && (k >= 64 || k == P))) {
                    __syncthreads();
                } else {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
            }
        }
    }

    // ---- 3. tau and Theta after each admission, the first failing one -----
    double loc[kSchedPer];
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e) {
        const int k = k0 + e;
        const float av = (e < E && k < N) ? __uint_as_float(~(uint32_t)(key[k] >> 32)) : 0.0f;
        run += (double)av;
        loc[e] = run;  // inclusive within the thread's run
    }
    // block exclusive scan of the thread totals
    const double incl = wave_incl_scan(run);
    if (lane == 63) wsum[wave] = incl;
    if (tid == 0) first_stop = 0x7fffffff;
    __syncthreads();
    double base = 0.0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    const double excl = base + (incl - run);
    const double theta0 = (R <= a.bmax) ? (double)R * (double)tab0 : 0.0;
    double th[kSchedPer];
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e) {
        const int k = k0 + e;
        const long B = (long)R + k + 1;  // batch after admitting candidates 0..k
        th[e] = (e < E && k < N && B <= a.bmax) ? ((double)R + excl + loc[e]) * (double)tab[e]
                                                : 0.0;
    }
    double lastv = 0.0;
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e)
        if (e == E - 1) lastv = th[e];
    last_theta[tid] = lastv;
    __syncthreads();
    int stop = 0x7fffffff;
    if (a.topk < 0) {
        double prev = tid == 0 ? theta0 : last_theta[tid - 1];
#pragma unroll
        for (int e = 0; e < kSchedPer; ++e) {
            const int k = k0 + e;
            if (e < E && k < N) {
                const long B = (long)R + k + 1;
                if ((B > a.bmax || !(th[e] > prev)) && stop == 0x7fffffff) stop = k;
                prev = th[e];
            }
        }
    } else {
        // top K: no comparison, only the table's end
        for (int e = 0; e < E; ++e) {
            const int k = k0 + e;
            if (k < N && (long)R + k + 1 > a.bmax && stop == 0x7fffffff) stop = k;
        }
    }
    stop = wave_min_i(stop);
    if (lane == 0 && stop != 0x7fffffff) atomicMin(&first_stop, stop);
    __syncthreads();
    int admitted = first_stop == 0x7fffffff ? N : first_stop;
    if (a.topk >= 0 && a.topk < admitted) admitted = a.topk;

    // ---- 4. lengths and the chosen Theta ------------------------------------
#pragma unroll
    for (int e = 0; e < kSchedPer; ++e) {
        const int k = k0 + e;
        if (e < E && k < admitted) {
            const uint32_t idx = (uint32_t)key[k];
            atomicMax(&len[idx / (uint32_t)G], (int)(idx % (uint32_t)G) + 1);
        }
        if (a.out_theta && e < E && k == admitted - 1) a.out_theta[0] = th[e];
    }
    if (a.out_theta && admitted == 0 && tid == 0) a.out_theta[0] = theta0;
    __syncthreads();
    for (int r = tid; r < R; r += kSchedThreads) a.out_len[r] = len[r];
}

}  // namespace sv

using namespace sv;

extern "C" {

size_t spec_schedule_workspace_bytes(void) { return sizeof(Control); }

int spec_schedule_verify_len(const float *confidence, const float *sps, int R, int gamma, int bmax,
                             int topk, int32_t *out_len, double *out_theta, void *workspace,
                             size_t workspace_bytes, void *stream) {
    if (R < 0 || gamma < 0 || bmax < 0) return SPEC_EINVAL;
    if ((long)R * gamma > kSchedMaxPool || R > kSchedMaxPool) return SPEC_EUNSUPPORTED;
    if (R == 0) return SPEC_OK;
    if (!sps || !out_len || (gamma > 0 && !confidence)) return SPEC_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < sizeof(Control))
        return SPEC_EWORKSPACE;
    SchedArgs a{};
    a.conf = confidence;
    a.sps = sps;
    a.R = R;
    a.gamma = gamma;
    a.bmax = bmax;
    a.topk = topk < 0 ? -1 : topk;
    int P = 1;
    while (P < R * gamma) P <<= 1;
    a.P = P;
    a.out_len = out_len;
    a.out_theta = out_theta;
    a.ctl = (Control *)workspace;
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
