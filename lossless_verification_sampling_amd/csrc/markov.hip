// markov.hip -- first-order Markov-head draft on gfx950.
//
// Method (DSpark paper guide, personal-site-bgy.pages.dev, "Markov head"):
// a parallel backbone gives base logits U_k for every draft position; a light
// serial head adds a transition bias that depends on the previously sampled
// token, p_k(v | x_0, x_<k) = softmax(U_k(v) + B(x_{k-1}, v)), with the V x V
// bias factored as B = W1 W2 (W1 in R^{V x r} used as an embedding lookup,
// W2 in R^{r x V} as a logit projection, r = 256) and x_0 the anchor token.
// Sampling is serial over k because x_k feeds the bias of step k+1.
//
// Per step k two launches:
//  * markov_logits_kernel: one workgroup per 128-logit tile of the vocabulary.
//    The tile of W2 ([256][128] bf16) is staged in LDS (transposed so each
//    lane reads 8 consecutive k of one column), the gathered rows W1[x_{k-1}]
//    of all requests feed v_mfma_f32_16x16x32_bf16 as the A operand, and the
//    epilogue adds U_k, stores the fp32 logits and reduces per-(request,
//    tile) softmax statistics (max and sum of 2^((l - m) s), or the argmax at
//    T = 0).  W2 is read once per step for all requests.
//  * markov_sample_kernel: one workgroup per request combines the tile
//    statistics, picks the tile holding u * total (inverse CDF in ascending
//    token id), re-reads that tile's 128 logits and finishes the draw.
#include <math.h>

#include "common.h"

namespace sv {

constexpr int kMkRank = 256;        // rank of W1 W2 (the pages' default r)
constexpr int kMkTile = 128;        // logits per tile
constexpr int kMkRows = 64;         // requests per MFMA row block (4 waves x 16)
constexpr int kMkLdsStride = kMkRank + 8;  // bf16 per LDS row (padding vs bank conflicts)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct MarkovArgs {
    const void *U;           // [R][gamma][V]
    const uint16_t *W1;      // [V][rank] bf16
    const uint16_t *W2;      // [rank][V] bf16
    const int32_t *anchor;   // [R]
    const float *temp;       // [R]
    const float *ud;         // [R][gamma]
    int R, gamma, V, ntiles;
    int k;                   // current step, 1..gamma
    int32_t *out_tok;        // [R][gamma]
    float *out_logits;       // [R][gamma][V]
    float2 *tstats;          // [R][ntiles]: (max, exp-sum) or (max, argmax bits)
    uint32_t *bad;           // [R] invalid-request flags
    Control *ctl;
};

__device__ __forceinline__ bool mk_temperature_ok(float T) {
    if (!(T >= 0.0f) || !(T <= 1e30f)) return false;
    return T == 0.0f || T >= 1e-30f;
}

template <typename TU>
__global__ void __launch_bounds__(kBlock) markov_logits_kernel(MarkovArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t w2t[kMkTile * kMkLdsStride];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int tile = blockIdx.x;
    const long v0 = (long)tile * kMkTile;
    const int V = a.V;

    // ---- stage W2[:, v0:v0+128] transposed: w2t[n][k] ------------------------
    // 256 rows of 128 bf16; thread t handles column group (t % 16) * 8 of rows
    // t / 16, t / 16 + 16, ...
    {
        const int cg = (tid & 15) * 8;
        for (int kk = tid >> 4; kk < kMkRank; kk += kBlock / 16) {
            const long base = (long)kk * V + v0 + cg;
            uint16_t v8[8];
            if ((V & 7) == 0 && v0 + cg + 8 <= V) {
                uint4 w = *reinterpret_cast<const uint4 *>(a.W2 + base);
                v8[0] = (uint16_t)w.x; v8[1] = (uint16_t)(w.x >> 16);
                v8[2] = (uint16_t)w.y; v8[3] = (uint16_t)(w.y >> 16);
                v8[4] = (uint16_t)w.z; v8[5] = (uint16_t)(w.z >> 16);
                v8[6] = (uint16_t)w.w; v8[7] = (uint16_t)(w.w >> 16);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) v8[q] = (v0 + cg + q < V) ? a.W2[base + q] : (uint16_t)0;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) w2t[(cg + q) * kMkLdsStride + kk] = v8[q];
        }
    }
    __syncthreads();

    const int col_in_blk = lane & 15;     // column within a 16-wide block
    const int kgrp = lane >> 4;           // which 8-wide k group of the 32
    const int k = a.k;

    for (int rb = 0; rb * kMkRows < a.R; ++rb) {
        // A operand rows of this wave: r = rb * 64 + wave * 16 + (lane % 16)
        const int ra = rb * kMkRows + wave * 16 + (lane & 15);
        int xprev = -1;
        if (ra < a.R) xprev = (k == 1) ? a.anchor[ra] : a.out_tok[(size_t)ra * a.gamma + (k - 2)];
        const bool xok = xprev >= 0 && xprev < V;
        f32x4_t acc[kMkTile / 16];
#pragma unroll
        for (int nb = 0; nb < kMkTile / 16; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int ks = 0; ks < kMkRank / 32; ++ks) {
            const int kk = ks * 32 + kgrp * 8;
            uint4 araw = make_uint4(0u, 0u, 0u, 0u);
            if (xok) araw = *reinterpret_cast<const uint4 *>(a.W1 + (long)xprev * kMkRank + kk);
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, araw);
#pragma unroll
            for (int nb = 0; nb < kMkTile / 16; ++nb) {
                const uint4 braw = *reinterpret_cast<const uint4 *>(
                    &w2t[(nb * 16 + col_in_blk) * kMkLdsStride + kk]);
                const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, braw);
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
            }
        }
        // ---- epilogue: D lane layout row = (lane / 16) * 4 + j, col = lane % 16
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = rb * kMkRows + wave * 16 + kgrp * 4 + j;
            const bool rok = r < a.R;
            const float T = rok ? a.temp[r] : 1.0f;
            const bool greedy = (T == 0.0f);
            const float s = (!greedy && mk_temperature_ok(T)) ? (float)(kLog2e / (double)T) : 1.0f;
            float lv[kMkTile / 16];
            float m = -__builtin_inff();
            int arg = 0x7fffffff, nanseen = 0;
#pragma unroll
            for (int nb = 0; nb < kMkTile / 16; ++nb) {
                const long v = v0 + nb * 16 + col_in_blk;
                float l = -__builtin_inff();
                if (rok && v < V) {
                    const TU *urow = (const TU *)a.U + ((long)r * a.gamma + (k - 1)) * V;
                    l = load_one(urow, v) + acc[nb][j];
                    a.out_logits[((long)r * a.gamma + (k - 1)) * V + v] = l;
                }
                lv[nb] = l;
                if (l != l) nanseen = 1;
                if (l > m) { m = l; arg = (int)v; }
            }
            // reduce over the 16 lanes sharing this row (lane bits 0..3)
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float m2 = __shfl_xor(m, o, 64);
                const int a2 = __shfl_xor(arg, o, 64);
                argmax_combine(m, arg, m2, a2);
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) nanseen |= __shfl_xor(nanseen, o, 64);
            float out1;
            if (greedy) {
                if (nanseen) m = __builtin_nanf("");
                out1 = __int_as_float(arg);
            } else {
                float e = 0.0f;
                if (m > -__builtin_inff()) {
#pragma unroll
                    for (int nb = 0; nb < kMkTile / 16; ++nb)
                        e += __builtin_amdgcn_exp2f((lv[nb] - m) * s);
                } else {
#pragma unroll
                    for (int nb = 0; nb < kMkTile / 16; ++nb)
                        if (lv[nb] != lv[nb]) e = lv[nb];
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) e += __shfl_xor(e, o, 64);
                out1 = e;
            }
            if (rok && col_in_blk == 0) a.tstats[(size_t)r * a.ntiles + tile] = make_float2(m, out1);
        }
    }
}

// One workgroup per request: tile choice, then the draw inside the tile.
__global__ void __launch_bounds__(kBlock) markov_sample_kernel(MarkovArgs a) {
    __shared__ BlockScratch bs;
    __shared__ int s_tok;
    __shared__ double s_t;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int k = a.k;
    const int V = a.V;
    const float T = a.temp[r];
    const int32_t anc = a.anchor[r];
    bool ok = mk_temperature_ok(T) && anc >= 0 && anc < V && a.bad[r] == 0u;
    const float u = a.ud[(size_t)r * a.gamma + (k - 1)];
    if (T != 0.0f && !(u >= 0.0f && u < 1.0f)) ok = false;
    const float2 *ts = a.tstats + (size_t)r * a.ntiles;
    int token = -1;

    if (ok && T == 0.0f) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff, nan = 0;
        for (int t = tid; t < a.ntiles; t += kBlock) {
            const float2 st = ts[t];
            if (st.x != st.x) nan = 1;
            argmax_combine(bv, bi, st.x, __float_as_int(st.y));
        }
        float dv = -__builtin_inff();
        int di = 0;
        block_argmax2(bv, bi, dv, di, bs);
        nan = block_max_i(nan, bs);
        ok = !nan && bv < __builtin_inff() && bi != 0x7fffffff;
        token = bi;
    } else if (ok) {
        const float s = (float)(kLog2e / (double)T);
        float M = -__builtin_inff(), dummy = -__builtin_inff();
        int bad = 0;
        for (int t = tid; t < a.ntiles; t += kBlock) {
            const float2 st = ts[t];
            M = fmaxf(M, st.x);
            if (st.y != st.y) bad = 1;
        }
        block_max2(M, dummy, bs);
        bad = block_max_i(bad, bs);
        ok = !bad && M > -__builtin_inff() && M < __builtin_inff();
        if (ok) {
            // tile masses in tile order, processed 256 tiles at a time
            double W = 0.0;
            for (int t0 = 0; t0 < a.ntiles; t0 += kBlock) {
                const int t = t0 + tid;
                double w = 0.0;
                if (t < a.ntiles) {
                    const float2 st = ts[t];
                    if (st.x > -__builtin_inff()) w = (double)st.y * exp2((double)(st.x - M) * (double)s);
                }
                double tot;
                (void)block_exclusive_scan(w, &tot, bs);
                W += tot;
            }
            const double tt = (double)u * W;
            double run = 0.0;
            int tile = -1, last_pos = -1;
            double tsel = 0.0;
            for (int t0 = 0; t0 < a.ntiles; t0 += kBlock) {
                const int t = t0 + tid;
                double w = 0.0;
                if (t < a.ntiles) {
                    const float2 st = ts[t];
                    if (st.x > -__builtin_inff()) w = (double)st.y * exp2((double)(st.x - M) * (double)s);
                }
                double tot;
                const double excl = run + block_exclusive_scan(w, &tot, bs);
                const int hit = block_min_i((t < a.ntiles && excl + w > tt) ? t : 0x7fffffff, bs);
                last_pos = max(last_pos, block_max_i(w > 0.0 ? t : -1, bs));
                if (hit != 0x7fffffff) {  // block-uniform
                    if (t == hit) s_t = tt - excl;
                    __syncthreads();
                    tile = hit;
                    tsel = s_t;
                    break;
                }
                run += tot;
            }
            if (tile < 0) {  // u * W at or past the total (rounding): last positive tile
                tile = last_pos;
                tsel = INFINITY;
            }
            if (tile < 0) tile = 0;  // unreachable: the tile holding the max has mass
            // draw inside the tile (one lane walks the 128 logits in order)
            if (tid == 0) {
                const float m = ts[tile].x;
                const long v0 = (long)tile * kMkTile;
                const float *lrow = a.out_logits + ((long)r * a.gamma + (k - 1)) * V;
                double cum = 0.0;
                int tok = -1, lastp = -1;
                for (int q = 0; q < kMkTile && v0 + q < V; ++q) {
                    const float e = (m > -__builtin_inff())
                                        ? __builtin_amdgcn_exp2f((lrow[v0 + q] - m) * s)
                                        : 0.0f;
                    if (e > 0.0f) lastp = (int)(v0 + q);
                    cum += (double)e * exp2((double)(m - M) * (double)s);
                    if (tok < 0 && cum > tsel) tok = (int)(v0 + q);
                }
                s_tok = (tok >= 0) ? tok : lastp;
            }
            __syncthreads();
            token = s_tok;
            ok = token >= 0;
        }
    }
    if (tid == 0) {
        if (!ok) a.bad[r] = 1u;
        a.out_tok[(size_t)r * a.gamma + (k - 1)] = ok ? token : -1;
        if (k == a.gamma && (a.bad[r] || !ok)) {
            for (int q = 0; q < a.gamma; ++q) a.out_tok[(size_t)r * a.gamma + q] = -1;
            atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
        }
    }
}

__global__ void markov_clear_kernel(uint32_t *bad, int R) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < R; i += gridDim.x * blockDim.x)
        bad[i] = 0u;
}

namespace {

size_t mk_round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct MkPlan {
    int ntiles;
    size_t off_stats, off_bad, bytes;
};

bool mk_plan(long R, long V, MkPlan &p) {
    p.ntiles = (int)((V + kMkTile - 1) / kMkTile);
    p.off_stats = sizeof(Control);
    p.off_bad = mk_round_up(p.off_stats + sizeof(float2) * (size_t)R * p.ntiles, 256);
    p.bytes = mk_round_up(p.off_bad + sizeof(uint32_t) * (size_t)R, 256);
    return true;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

size_t spec_markov_workspace_bytes(int R, int gamma, int V, int rank) {
    if (R < 0 || gamma < 0 || V < 1 || V > SPEC_MAX_VOCAB || rank != kMkRank) return 0;
    MkPlan p;
    mk_plan(R > 0 ? R : 1, V, p);
    return p.bytes;
}

int spec_markov_draft_sample(const void *U, int u_dtype, const void *W1, const void *W2,
                             int w_dtype, const int32_t *anchor, const float *temperature,
                             const float *u_draft, int R, int gamma, int V, int rank,
                             int32_t *out_draft_tokens, float *out_draft_logits, void *workspace,
                             size_t workspace_bytes, void *stream) {
    if (R < 0 || gamma < 0 || V < 1) return SPEC_EINVAL;
    if ((u_dtype != SPEC_F32 && u_dtype != SPEC_BF16) || w_dtype != SPEC_BF16) return SPEC_EDTYPE;
    if (rank != kMkRank || V > SPEC_MAX_VOCAB) return SPEC_EUNSUPPORTED;
    if (R == 0 || gamma == 0) return SPEC_OK;
    if (!U || !W1 || !W2 || !anchor || !temperature || !u_draft || !out_draft_tokens ||
        !out_draft_logits)
        return SPEC_EINVAL;
    if (((uintptr_t)W1 & 15u) || ((uintptr_t)W2 & 15u)) return SPEC_EINVAL;
    MkPlan p;
    mk_plan(R, V, p);
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < p.bytes)
        return SPEC_EWORKSPACE;
    char *ws = (char *)workspace;
    MarkovArgs a{};
    a.U = U;
    a.W1 = (const uint16_t *)W1;
    a.W2 = (const uint16_t *)W2;
    a.anchor = anchor;
    a.temp = temperature;
    a.ud = u_draft;
    a.R = R;
    a.gamma = gamma;
    a.V = V;
    a.ntiles = p.ntiles;
    a.out_tok = out_draft_tokens;
    a.out_logits = out_draft_logits;
    a.tstats = (float2 *)(ws + p.off_stats);
    a.bad = (uint32_t *)(ws + p.off_bad);
    a.ctl = (Control *)ws;
    note_workspace_clean(workspace, sizeof(Control));
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(markov_clear_kernel, dim3((R + kBlock - 1) / kBlock), dim3(kBlock), 0, st,
                       a.bad, R);
    for (int k = 1; k <= gamma; ++k) {
        a.k = k;
        if (u_dtype == SPEC_BF16)
            hipLaunchKernelGGL(markov_logits_kernel<uint16_t>, dim3(p.ntiles), dim3(kBlock), 0, st,
                               a);
        else
            hipLaunchKernelGGL(markov_logits_kernel<float>, dim3(p.ntiles), dim3(kBlock), 0, st, a);
        hipLaunchKernelGGL(markov_sample_kernel, dim3(R), dim3(kBlock), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
