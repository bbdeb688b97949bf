// sts.hip -- sequential temperature scaling (STS) of the confidence head on
// gfx950.
//
// Method (DSpark paper guide, personal-site-bgy.pages.dev, the
// confidence-head section, "STS"): the head's per-position scores are
// calibrated after training on a held-out set, left to right: for position k
// a one-dimensional grid search picks the temperature t_k that minimises the
// expected calibration error of the cumulative probabilities
// a_k = c_1(t_1) ... c_k(t_k), c(t) = sigmoid(z / t), with the positions
// before k fixed at their chosen temperatures.  The label of a_k is the
// event that positions 1..k were all accepted ([A >= k] for a block's
// accepted prefix length A), and ECE over `bins` equal-width bins is
// sum_m |sum_{n in bin m} (a_n - y_n)| / N.  Ties go to the first grid point.
//
// Per position, three launches on the caller's stream:
//  1. sts_hist_kernel: workgroup (tile of 512 held-out blocks, 64 grid
//     points).  The tile's (z_k, a_{k-1}, y_k) are staged in LDS; a_{k-1} is
//     made there from a_{k-2} and the previous position's chosen
//     temperature, and the first grid block writes it back (two buffers, so
//     no workgroup reads what another writes).  Lane j of every wave takes
//     grid point j and wave w the tile's blocks w, w + 4, ...; each thread
//     adds a - y into its own LDS column of bin sums (fp64, blocks in order),
//     the four waves' columns are added in wave order, and the tile's sums go
//     to the workspace.
//  2. sts_reduce_kernel: one wave per (grid point, bin) adds the tiles' sums
//     (lane runs in tile order, then a fixed DPP tree).
//  3. sts_select_kernel: one workgroup computes the ECE per grid point, the
//     first minimum and the position's outputs.  (Folding this into the
//     reduce launch's last workgroup needs a device-scope fence in every
//     workgroup, which costs more than the launch.)
// All sums have a fixed order, so repeated calls give identical results.
#include <math.h>

#include "common.h"

namespace sv {

constexpr int kStsTile = 512;   // held-out blocks per workgroup of the histogram
constexpr int kStsGrid = 64;    // grid points per workgroup (one per lane)
constexpr int kStsMaxBins = SPEC_STS_MAX_BINS;
constexpr int kStsMaxGrid = SPEC_STS_MAX_GRID;

struct StsArgs {
    const float *z;        // [N][gamma] raw confidence logits
    const int32_t *alen;   // [N] accepted prefix lengths
    const double *grid;    // [G] temperatures
    int N, gamma, G, bins, ntiles, k;  // k: the position (0-based)
    double *abuf;          // [2][N] cumulative probabilities: a_m in buffer m & 1
    double *part;          // [G * bins][ntiles] per-tile bin sums of a - y
    double *sums;          // [G * bins] bin sums
    uint32_t *bad;         // input fault flag (0 / 1)
    double *out_t;         // [gamma]
    double *out_ece;       // [gamma]
    double *out_curve;     // [gamma][G] or null
    Control *ctl;
};

// 1 / d for d in [1, inf]: the hardware reciprocal refined by two Newton
// steps (d = inf gives 0).
__device__ __forceinline__ double sts_inv1p(double d) {
    double r = __builtin_amdgcn_rcp(d);
    r = fma(r, fma(-d, r, 1.0), r);
    r = fma(r, fma(-d, r, 1.0), r);
    return d < INFINITY ? r : 0.0;
}

// sigmoid(z / t) with rt = 1 / t.
__device__ __forceinline__ double sts_sigmoid(double z, double rt) {
    return sts_inv1p(1.0 + exp(-(z * rt)));
}

__device__ __forceinline__ int sts_bin(double a, int bins) {
    const int m = (int)floor(a * (double)bins);
    return m < bins - 1 ? (m > 0 ? m : 0) : bins - 1;
}

__global__ void sts_clear_kernel(uint32_t *bad) { atomic_store_u32(bad, 0u); }

// a_{-1} = 1 for every block (buffer 1), and the inputs checked: every logit
// finite, every accepted length in [0, gamma].
__global__ void __launch_bounds__(kBlock) sts_init_kernel(StsArgs a) {
    const long n = (long)blockIdx.x * kBlock + threadIdx.x;
    if (n >= a.N) return;
    a.abuf[a.N + n] = 1.0;
    bool ok = a.alen[n] >= 0 && a.alen[n] <= a.gamma;
    for (int k = 0; k < a.gamma; ++k) {
        const float z = a.z[(size_t)n * a.gamma + k];
        ok = ok && (z - z == 0.0f);
    }
    if (!ok) atomic_or_u32(a.bad, 1u);
}

__global__ void __launch_bounds__(kBlock) sts_hist_kernel(StsArgs a) {
    extern __shared__ double sh[];
    double *acc = sh;                                   // [bins][kBlock]
    double *ap = sh + (size_t)a.bins * kBlock;          // [kStsTile]
    float *zt = (float *)(ap + kStsTile);               // [kStsTile]
    float *yt = zt + kStsTile;                          // [kStsTile]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long n0 = (long)blockIdx.x * kStsTile;
    const int nt = (int)min((long)kStsTile, (long)a.N - n0);
    // a_{k-1} = a_{k-2} sigmoid(z_{k-1} / t_{k-1}), a_{-1} = 1
    const double rtp = a.k > 0 ? 1.0 / a.out_t[a.k - 1] : 0.0;
    const double *src = a.abuf + (size_t)(a.k & 1) * a.N;        // a_{k-2}
    double *dst = a.abuf + (size_t)((a.k + 1) & 1) * a.N;        // a_{k-1}
    for (int i = tid; i < nt; i += kBlock) {
        const long n = n0 + i;
        double av = 1.0;
        if (a.k > 0) {
            av = src[n] * sts_sigmoid((double)a.z[(size_t)n * a.gamma + a.k - 1], rtp);
            if (blockIdx.y == 0) dst[n] = av;
        }
        ap[i] = av;
        zt[i] = a.z[(size_t)n * a.gamma + a.k];
        yt[i] = a.alen[n] >= a.k + 1 ? 1.0f : 0.0f;
    }
    for (int m = 0; m < a.bins; ++m) acc[m * kBlock + tid] = 0.0;
    __syncthreads();
    const int g = blockIdx.y * kStsGrid + lane;
    const double rt = 1.0 / (g < a.G ? a.grid[g] : 1.0);
    for (int i = wave; i < nt; i += kWaves) {
        const double av = ap[i] * sts_sigmoid((double)zt[i], rt);
        const int m = sts_bin(av, a.bins);
        acc[m * kBlock + tid] += av - (double)yt[i];
    }
    __syncthreads();
    // the four waves' rows in wave order; wave w writes bins w, w + 4, ...
    if (g < a.G) {
        for (int m = wave; m < a.bins; m += kWaves) {
            const double s = ((acc[m * kBlock + lane] + acc[m * kBlock + 64 + lane]) +
                              acc[m * kBlock + 128 + lane]) +
                             acc[m * kBlock + 192 + lane];
            a.part[((size_t)g * a.bins + m) * a.ntiles + blockIdx.x] = s;
        }
    }
}

// The position's choice: ECE per grid point, the first minimum, the outputs
// (one workgroup; grid points g = tid, tid + kBlock, ...).
__global__ void __launch_bounds__(kBlock) sts_select_kernel(StsArgs a) {
    __shared__ double best_e[kWaves];
    __shared__ int best_i[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int gbad = atomic_load_u32(a.bad) != 0u;
    double v = INFINITY;
    int idx = 0x7fffffff;
    for (int g = tid; g < a.G; g += kBlock) {
        const double t = a.grid[g];
        gbad |= !(t > 0.0 && t < INFINITY);
        double s = 0.0;
        for (int m = 0; m < a.bins; ++m) s += fabs(a.sums[(size_t)g * a.bins + m]);
        const double e = s / (double)a.N;
        if (a.out_curve) a.out_curve[(size_t)a.k * a.G + g] = e;
        if (e < v) {  // g ascending: the first minimum of this thread's points
            v = e;
            idx = g;
        }
    }
    if (__syncthreads_or(gbad)) {
        for (int g = tid; g < a.G; g += kBlock)
            if (a.out_curve) a.out_curve[(size_t)a.k * a.G + g] = NAN;
        if (tid == 0) {
            a.out_t[a.k] = NAN;
            a.out_ece[a.k] = NAN;
            atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
            atomic_or_u32(a.bad, 1u);
        }
        return;
    }
    // first minimum: the smallest (ECE, index) pair
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double v2 = __shfl_xor(v, o, 64);
        const int i2 = __shfl_xor(idx, o, 64);
        if (v2 < v || (v2 == v && i2 < idx)) {
            v = v2;
            idx = i2;
        }
    }
    if (lane == 0) {
        best_e[wave] = v;
        best_i[wave] = idx;
    }
    __syncthreads();
    if (tid == 0) {
        double bv = best_e[0];
        int bi = best_i[0];
        for (int w = 1; w < kWaves; ++w) {
            if (best_e[w] < bv || (best_e[w] == bv && best_i[w] < bi)) {
                bv = best_e[w];
                bi = best_i[w];
            }
        }
        a.out_t[a.k] = a.grid[bi];
        a.out_ece[a.k] = bv;
    }
}

// One wave per (grid point, bin): lane j adds tiles j, j + 64, ... in order,
// then the wave's fixed reduction tree.
__global__ void __launch_bounds__(kBlock) sts_reduce_kernel(StsArgs a) {
    const long w = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w >= (long)a.G * a.bins) return;
    const double *p = a.part + (size_t)w * a.ntiles;
    double s = 0.0;
    for (int i = lane; i < a.ntiles; i += 64) s += p[i];
    s = wave_sum(s);
    if (lane == 0) a.sums[w] = s;
}

struct StsPlan {
    int ntiles;
    size_t off_bad, off_ap, off_part, off_sums, bytes;
};

size_t sts_round(size_t x) { return (x + 255) / 256 * 256; }

void sts_plan(long N, int G, int bins, StsPlan &p) {
    p.ntiles = (int)((N + kStsTile - 1) / kStsTile);
    p.off_bad = sizeof(Control);
    p.off_ap = sts_round(p.off_bad + 4);
    p.off_part = sts_round(p.off_ap + 16 * (size_t)N);
    p.off_sums = sts_round(p.off_part + 8 * (size_t)G * bins * p.ntiles);
    p.bytes = sts_round(p.off_sums + 8 * (size_t)G * bins);
}

}  // namespace sv

using namespace sv;

extern "C" {

size_t spec_sts_workspace_bytes(int N, int gamma, int G, int bins) {
    if (N < 1 || gamma < 0 || G < 1 || G > kStsMaxGrid || bins < 1 || bins > kStsMaxBins ||
        (long)N > SPEC_STS_MAX_BLOCKS)
        return 0;
    StsPlan p;
    sts_plan(N, G, bins, p);
    return p.bytes;
}

int spec_sts_calibrate(const float *conf_logits, const int32_t *accepted_len, const double *grid,
                       int N, int gamma, int G, int bins, double *out_temperature,
                       double *out_ece, double *out_curve, void *workspace,
                       size_t workspace_bytes, void *stream) {
    if (N < 0 || gamma < 0 || G < 1 || bins < 1) return SPEC_EINVAL;
    if (G > kStsMaxGrid || bins > kStsMaxBins || (long)N > SPEC_STS_MAX_BLOCKS)
        return SPEC_EUNSUPPORTED;
    if (N == 0 || gamma == 0) return SPEC_OK;
    if (!conf_logits || !accepted_len || !grid || !out_temperature || !out_ece) return SPEC_EINVAL;
    StsPlan p;
    sts_plan(N, G, bins, p);
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < p.bytes)
        return SPEC_EWORKSPACE;
    char *ws = (char *)workspace;
    StsArgs a{};
    a.z = conf_logits;
    a.alen = accepted_len;
    a.grid = grid;
    a.N = N;
    a.gamma = gamma;
    a.G = G;
    a.bins = bins;
    a.ntiles = p.ntiles;
    a.abuf = (double *)(ws + p.off_ap);
    a.part = (double *)(ws + p.off_part);
    a.sums = (double *)(ws + p.off_sums);
    a.bad = (uint32_t *)(ws + p.off_bad);
    a.out_t = out_temperature;
    a.out_ece = out_ece;
    a.out_curve = out_curve;
    a.ctl = (Control *)ws;
    hipStream_t st = (hipStream_t)stream;
    const dim3 nblk((unsigned)((N + kBlock - 1) / kBlock));
    const dim3 hgrid((unsigned)p.ntiles, (unsigned)((G + kStsGrid - 1) / kStsGrid));
    const size_t lds = 8 * (size_t)bins * kBlock + (8 + 4 + 4) * (size_t)kStsTile;
    const dim3 rgrid((unsigned)(((long)G * bins + kWaves - 1) / kWaves));
    hipLaunchKernelGGL(sts_clear_kernel, dim3(1), dim3(1), 0, st, a.bad);
    hipLaunchKernelGGL(sts_init_kernel, nblk, dim3(kBlock), 0, st, a);
    for (int k = 0; k < gamma; ++k) {
        a.k = k;
        hipLaunchKernelGGL(sts_hist_kernel, hgrid, dim3(kBlock), lds, st, a);
        hipLaunchKernelGGL(sts_reduce_kernel, rgrid, dim3(kBlock), 0, st, a);
        hipLaunchKernelGGL(sts_select_kernel, dim3(1), dim3(kBlock), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
