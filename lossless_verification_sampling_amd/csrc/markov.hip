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
//  * markov_logits_kernel: one workgroup per 64-logit tile of the vocabulary.
//    The tile of W2 ([256][64] bf16) is staged in LDS transposed, w2t[n][k],
//    by loading 8x8 blocks, transposing them in registers and writing 16-byte
//    rows.  The product b[v][r] = sum_k W2[k][v] W1[x_r][k] runs on
//    v_mfma_f32_16x16x32_bf16 with the W2 tile as the A operand (16 vocabulary
//    rows per block) and the gathered rows W1[x_{k-1}] as B (16 requests per
//    block), so that each lane ends with four consecutive vocabulary entries
//    of one request: U is read and the fp32 logits written 8 and 16 bytes at
//    a time, and the per-(request, tile) softmax statistics (max and sum of
//    2^((l - m) s), or the argmax at T = 0) reduce inside the wave.  W2 is
//    read once per step for all requests.
//  * markov_sample_kernel: one workgroup per request combines the tile
//    statistics (block maximum and a block scan over the threads' runs of
//    tiles), picks the tile holding u * total (inverse CDF in ascending
//    token id), and its first wave re-reads that tile's 64 logits and
//    finishes the draw with a wave scan.
#include <math.h>
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "common.h"

namespace sv {

constexpr int kMkRank = 256;        // rank of W1 W2 (the pages' default r)
constexpr int kMkTile = 64;         // logits per tile (one workgroup each)
constexpr int kMkRows = 64;         // requests per MFMA row block (4 waves x 16)
constexpr int kMkLdsStride = kMkRank + 8;  // bf16 per LDS row (padding vs bank conflicts)
constexpr int kMkPipeTiles = 8;     // tiles per workgroup of the persistent logits launch

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Offset (bf16 elements) of the 16-byte piece k = 8 u .. 8 u + 7 of row n of
// the transposed W2 tile in LDS.  The row stride of 264 elements (33 pieces)
// spreads the consecutive rows an MFMA operand read touches over the banks.
// SW: the piece index is XOR-ed with bits 3..5 of the row, which does the
// same for the persistent launch's staging writes (16 lanes per pass, rows 8
// apart: without it each write was an 8-way bank conflict, and
// SQ_LDS_BANK_CONFLICT fell from 4.65e6 to 1.03e6 per logits launch).  The
// per-tile launch keeps the plain map: with it the RNN head's three-pass
// tiles ran 459 us per call against 434.
template <bool SW>
__device__ __forceinline__ int w2t_off(int n, int u) {
    return n * kMkLdsStride + 8 * (SW ? (u ^ ((n >> 3) & 7)) : u);
}
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
    int vec;                 // U rows and logit rows allow 4-wide loads and stores
    const uint16_t *bsplit;  // RNN head: [3][R][rank] bf16 parts of the state (B rows)
    int tile0;               // first tile of the launch
    int tile1;               // end of the launch's tiles (persistent launch)
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

// 8 x 8 block transpose of bf16 pairs: r[j] holds row j (8 values, two per
// word); c[i] gets column i (the 8 rows' values, two per word, row order).
__device__ __forceinline__ void transpose8x8(const uint4 (&r)[8], uint4 (&c)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint4 &lo = r[2 * d], &hi = r[2 * d + 1];
            const uint32_t a = (i >> 1) == 0 ? lo.x : (i >> 1) == 1 ? lo.y : (i >> 1) == 2 ? lo.z : lo.w;
            const uint32_t b = (i >> 1) == 0 ? hi.x : (i >> 1) == 1 ? hi.y : (i >> 1) == 2 ? hi.z : hi.w;
            w[d] = (i & 1) ? ((b & 0xffff0000u) | (a >> 16)) : ((b << 16) | (a & 0xffffu));
        }
        c[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Per-lane operands of one 16-request block: the request, its W1 row slices
// (the B operand for the 8 k steps) and its U values for the tile.
template <typename TU> struct MkLane;
template <> struct MkLane<uint16_t> {
    uint2 u[kMkTile / 16];  // 4 bf16 of U per vocabulary block
};
template <> struct MkLane<float> {
    float4 u[kMkTile / 16];
};

// The previous token of request r (the anchor at the first step); -1 for a
// request outside the batch.
__device__ __forceinline__ int mk_prev_token(const MarkovArgs &a, int r) {
    if (r >= a.R) return -1;
    return (a.k == 1) ? a.anchor[r] : a.out_tok[(size_t)r * a.gamma + (a.k - 2)];
}

// U values of request r for this lane's 4 vocabulary entries in each block.
template <typename TU, bool FULL>
__device__ __forceinline__ void mk_load_u(const MarkovArgs &a, int r, long v0, int kgrp,
                                          MkLane<TU> &ln) {
    const int V = a.V;
    const TU *urow = (const TU *)a.U + ((long)(r < a.R ? r : 0) * a.gamma + (a.k - 1)) * V;
#pragma unroll
    for (int vb = 0; vb < kMkTile / 16; ++vb) {
        const long v = v0 + vb * 16 + kgrp * 4;
        if constexpr (sizeof(TU) == 2) {
            if constexpr (FULL) {
                ln.u[vb] = *reinterpret_cast<const uint2 *>(urow + v);
            } else {
                uint32_t h[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) h[j] = (v + j < V) ? (uint32_t)urow[v + j] : 0u;
                ln.u[vb] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        } else {
            if constexpr (FULL) {
                ln.u[vb] = *reinterpret_cast<const float4 *>(urow + v);
            } else {
                float h[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) h[j] = (v + j < V) ? urow[v + j] : 0.0f;
                ln.u[vb] = make_float4(h[0], h[1], h[2], h[3]);
            }
        }
    }
}

// The B operand of the 8 k steps: W1[xprev][ks * 32 + kgrp * 8 .. + 8]
// (zero for an invalid previous token).
__device__ __forceinline__ void mk_load_w1(const MarkovArgs &a, int xprev, int kgrp,
                                           uint4 (&b)[kMkRank / 32]) {
    const bool xok = xprev >= 0 && xprev < a.V;
    const uint16_t *w1 = a.W1 + (long)(xok ? xprev : 0) * kMkRank + kgrp * 8;
#pragma unroll
    for (int ks = 0; ks < kMkRank / 32; ++ks) {
        b[ks] = *reinterpret_cast<const uint4 *>(w1 + ks * 32);
        if (!xok) b[ks] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// The B operand of the 8 k steps for request r: the gathered row W1[xprev]
// (Markov head, NSPLIT = 1), or bf16 part sp of the request's state (RNN
// head, NSPLIT = 3; the fp32 state is the sum of its three parts).
template <int NSPLIT>
__device__ __forceinline__ void mk_load_b(const MarkovArgs &a, int xprev, int r, int sp, int kgrp,
                                          uint4 (&b)[kMkRank / 32]) {
    if constexpr (NSPLIT == 1) {
        mk_load_w1(a, xprev, kgrp, b);
    } else {
        const bool rok = r < a.R;
        const uint16_t *row = a.bsplit + ((size_t)sp * a.R + (rok ? r : 0)) * kMkRank + kgrp * 8;
        const uint32_t keep = rok ? ~0u : 0u;
#pragma unroll
        for (int ks = 0; ks < kMkRank / 32; ++ks) {
            const uint4 w = *reinterpret_cast<const uint4 *>(row + ks * 32);
            b[ks] = make_uint4(w.x & keep, w.y & keep, w.z & keep, w.w & keep);
        }
    }
}

__device__ __forceinline__ void mk_unpack_u(const uint2 &w, float (&o)[4]) {
    o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x); o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
}
__device__ __forceinline__ void mk_unpack_u(const float4 &w, float (&o)[4]) {
    o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
}

// Epilogue of one (request, tile) for the lanes of request r (temperature
// T): acc[vb][j] = b[v][r] for v = v0 + vb * 16 + kgrp * 4 + j.  The logits
// U + b are written out, and the tile's statistics of the request (max and
// the sum of 2^((l - max) s), or the argmax at T = 0) reduce over the four
// lanes that share it.  ALL: every lane's request exists (rok), and the four
// lanes of a request all store its statistics (the same value), so that no
// store sits behind a branch.
template <typename TU, bool FULL, bool ALL = false>
__device__ __forceinline__ void mk_epilogue(const MarkovArgs &a, int r, bool rok, float T,
                                            int tile, long v0, int kgrp,
                                            const f32x4_t (&acc)[kMkTile / 16],
                                            const MkLane<TU> &ln) {
    const int V = a.V;
    const bool greedy = (T == 0.0f);
    const float s = (!greedy && mk_temperature_ok(T)) ? (float)(kLog2e / (double)T) : 1.0f;
    float *lrow = a.out_logits + ((long)(rok ? r : 0) * a.gamma + (a.k - 1)) * V;
    float lv[kMkTile / 16][4];
    float m = -__builtin_inff();
    int arg = 0x7fffffff, nanseen = 0;
#pragma unroll
    for (int vb = 0; vb < kMkTile / 16; ++vb) {
        const long v = v0 + vb * 16 + kgrp * 4;
        float u4[4];
        mk_unpack_u(ln.u[vb], u4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float l = (rok && v + j < V) ? u4[j] + acc[vb][j] : -__builtin_inff();
            lv[vb][j] = l;
            if (l != l) nanseen = 1;
            if (l > m) { m = l; arg = (int)(v + j); }
        }
        if (ALL || rok) {
            if constexpr (FULL) {
                *reinterpret_cast<float4 *>(lrow + v) =
                    make_float4(lv[vb][0], lv[vb][1], lv[vb][2], lv[vb][3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (v + j < V) lrow[v + j] = lv[vb][j];
            }
        }
    }
    // reduce over the 4 lanes sharing this request (lane bits 4..5): the
    // partner across rows, then across halves
    auto pair_max = [&](auto tag) {
        constexpr int P = decltype(tag)::value;
        uint32_t m0, m1, a0, a1, n0, n1;
        lane_pair<P>(__float_as_uint(m), m0, m1);
        lane_pair<P>((uint32_t)arg, a0, a1);
        lane_pair<P>((uint32_t)nanseen, n0, n1);
        m = __uint_as_float(m0);
        arg = (int)a0;
        argmax_combine(m, arg, __uint_as_float(m1), (int)a1);
        nanseen = (int)(n0 | n1);
    };
    pair_max(std::integral_constant<int, 16>{});
    pair_max(std::integral_constant<int, 32>{});
    float out1;
    if (greedy) {
        if (nanseen) m = __builtin_nanf("");
        out1 = __int_as_float(arg);
    } else {
        float e = 0.0f;
        if (m > -__builtin_inff()) {
#pragma unroll
            for (int vb = 0; vb < kMkTile / 16; ++vb)
#pragma unroll
                for (int j = 0; j < 4; ++j) e += __builtin_amdgcn_exp2f((lv[vb][j] - m) * s);
        } else {
#pragma unroll
            for (int vb = 0; vb < kMkTile / 16; ++vb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (lv[vb][j] != lv[vb][j]) e = lv[vb][j];
        }
        uint32_t e0, e1;
        lane_pair<16>(__float_as_uint(e), e0, e1);
        e = __uint_as_float(e0) + __uint_as_float(e1);
        lane_pair<32>(__float_as_uint(e), e0, e1);
        e = __uint_as_float(e0) + __uint_as_float(e1);
        out1 = e;
    }
    if (ALL || (rok && kgrp == 0)) a.tstats[(size_t)r * a.ntiles + tile] = make_float2(m, out1);
}

// FULL: every tile of the launch lies inside the row, V is a multiple of 8
// (16-byte aligned W2 rows) and the U and logit rows allow 4-wide accesses,
// so every load and store is a vector; otherwise (odd V, the ragged last
// tile, unaligned U or logits) they are guarded scalars.
template <typename TU, bool FULL, int NSPLIT>
__global__ void __launch_bounds__(kBlock, 4) markov_logits_kernel(MarkovArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t w2t[kMkTile * kMkLdsStride];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int tile = a.tile0 + (int)blockIdx.x;
    const long v0 = (long)tile * kMkTile;
    const int V = a.V;
    const int col = lane & 15;   // request within the wave's 16 / vocabulary row within A
    const int kgrp = lane >> 4;  // which 8-wide k group of the 32

    // ---- issue every load of the first request block up front ---------------
    // W2 block (k0.., n0..): 8 consecutive threads read one 128-byte row piece
    const int k0 = (tid >> 3) * 8, n0 = (tid & 7) * 8;
    uint4 rw[8];
    if constexpr (FULL) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            rw[j] = *reinterpret_cast<const uint4 *>(a.W2 + (long)(k0 + j) * V + v0 + n0);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t w[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const long c = v0 + n0 + 2 * d;
                const uint32_t x0 = c < V ? a.W2[(long)(k0 + j) * V + c] : 0u;
                const uint32_t x1 = c + 1 < V ? a.W2[(long)(k0 + j) * V + c + 1] : 0u;
                w[d] = x0 | (x1 << 16);
            }
            rw[j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    int xprev = mk_prev_token(a, wave * 16 + col);
    MkLane<TU> ln;
    mk_load_u<TU, FULL>(a, wave * 16 + col, v0, kgrp, ln);
    // the W1 operand too, where registers allow (the guarded variant's
    // scalar staging needs them; it loads W1 after the barrier)
    uint4 bop[kMkRank / 32];
    if constexpr (FULL) mk_load_b<NSPLIT>(a, xprev, wave * 16 + col, 0, kgrp, bop);

    // ---- stage W2[:, v0:v0+64] transposed: w2t[n][k] -------------------------
    {
        uint4 cw[8];
        transpose8x8(rw, cw);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4 *>(&w2t[w2t_off<false>(n0 + i, k0 / 8)]) = cw[i];
    }
    __syncthreads();

    for (int rb = 0; rb * kMkRows < a.R; ++rb) {
        const int r = rb * kMkRows + wave * 16 + col;
        const bool rok = r < a.R;
        // keeps the tile's LDS reads inside the loop: hoisted out of it they
        // would hold the whole 32 KB A operand in registers
        asm volatile("" ::: "memory");
        if (rb > 0) {
            xprev = mk_prev_token(a, r);
            mk_load_u<TU, FULL>(a, r, v0, kgrp, ln);
        }
        if (rb > 0 || !FULL) mk_load_b<NSPLIT>(a, xprev, r, 0, kgrp, bop);
        // b[v][r] = sum_k W2[k][v] B_r[k]: A = the W2 tile (16 vocabulary rows
        // per block), B = 16 gathered W1 rows (Markov head) or the bf16 parts
        // of 16 states, one after the other (RNN head)
        f32x4_t acc[kMkTile / 16];
#pragma unroll
        for (int vb = 0; vb < kMkTile / 16; ++vb) acc[vb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < NSPLIT; ++sp) {
            if (sp > 0) {
                asm volatile("" ::: "memory");
                mk_load_b<NSPLIT>(a, xprev, r, sp, kgrp, bop);
            }
#pragma unroll
            for (int ks = 0; ks < kMkRank / 32; ++ks) {
                const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bop[ks]);
#pragma unroll
                for (int vb = 0; vb < kMkTile / 16; ++vb) {
                    const uint4 araw = *reinterpret_cast<const uint4 *>(
                        &w2t[w2t_off<false>(vb * 16 + col, ks * 4 + kgrp)]);
                    acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, araw), bv, acc[vb], 0, 0, 0);
                }
            }
        }
        // ---- epilogue: acc[vb][j] = b[v][r], v = v0 + vb * 16 + kgrp * 4 + j
        mk_epilogue<TU, FULL>(a, r, rok, rok ? a.temp[r] : 1.0f, tile, v0, kgrp, acc, ln);
    }
}

// The common case of markov_logits_kernel (whole tiles in 16-byte aligned
// rows, exactly 64 requests, the Markov head) as a persistent launch over
// wide tiles of 64 H ids (H 64-id tiles side by side, 256 H threads; wave w
// takes requests 16 (w % 4) .. + 15 and the 64-id part w / 4): workgroup g
// takes wide tiles tile0 + g, + G, ... < tile1 (in units of 64 H ids).  The
// W2 loads run two tiles ahead of the product and epilogue and the U loads
// one (two register sets taken in turn, each reloaded only after its last
// use), the tile's W2 block alternates between two shared-memory buffers
// (one barrier per tile), and the gathered W1 rows are loaded once.  Every
// load and store is unconditional (a tile past the end reads the last one
// again and is not used) and the tile loop is unrolled, so that the
// compiler's wait counts stay exact and a tile's stores never hold up the
// next tiles' loads.  Wider tiles read W2 and U and write the logits in
// longer row pieces (128 H bytes of W2 and U, 256 H of logits).  Same
// arithmetic, in the same order, as markov_logits_kernel; the statistics
// stay per 64-id tile.
template <typename TU, int H>
__global__ void __launch_bounds__(kBlock * H, 2 / H) markov_logits_pipe_kernel(MarkovArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t mk_dyn[];
    constexpr int TW = kMkTile * H;  // ids per wide tile
    uint16_t *const w2t[2] = {mk_dyn, mk_dyn + TW * kMkLdsStride};
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kgrp = lane >> 4;
    const int part = wave >> 2;                    // 64-id part of the wide tile
    const int k0 = (tid / (TW / 8)) * 8, n0 = (tid % (TW / 8)) * 8;
    const int r = (wave & 3) * 16 + col;
    const long V = a.V;
    const int G = (int)gridDim.x;
    const int tend = a.tile1;
    int tile = a.tile0 + (int)blockIdx.x;
    auto tile_v0 = [&](int t) { return (long)(t < tend ? t : tend - 1) * TW; };
    auto fetch_w2 = [&](int t, uint4 (&rw)[8]) {
        const long v0 = tile_v0(t);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            rw[j] = *reinterpret_cast<const uint4 *>(a.W2 + (long)(k0 + j) * V + v0 + n0);
    };
    auto fetch_u = [&](int t, MkLane<TU> &u) {
        mk_load_u<TU, true>(a, r, tile_v0(t) + part * kMkTile, kgrp, u);
    };
    auto stage = [&](int buf, const uint4 (&rw)[8]) {
        uint4 cw[8];
        transpose8x8(rw, cw);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4 *>(&w2t[buf][w2t_off<true>(n0 + i, k0 / 8)]) = cw[i];
    };
    // the request's operands first (their waits then leave the tile loads
    // in flight): the gathered W1 row and the temperature
    const int xprev = mk_prev_token(a, r);
    const float T = a.temp[r];
    uint4 bop[kMkRank / 32];
    mk_load_b<1>(a, xprev, r, 0, kgrp, bop);
    auto product = [&](int buf, int t, const MkLane<TU> &u) {
        f32x4_t acc[kMkTile / 16];
#pragma unroll
        for (int vb = 0; vb < kMkTile / 16; ++vb) acc[vb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kMkRank / 32; ++ks) {
            const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bop[ks]);
#pragma unroll
            for (int vb = 0; vb < kMkTile / 16; ++vb) {
                const uint4 araw = *reinterpret_cast<const uint4 *>(
                    &w2t[buf][w2t_off<true>(part * kMkTile + vb * 16 + col, ks * 4 + kgrp)]);
                acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, araw), bv, acc[vb], 0, 0, 0);
            }
        }
        mk_epilogue<TU, true, true>(a, r, true, T, t * H + part,
                                    (long)t * TW + part * kMkTile, kgrp, acc, u);
    };
    uint4 ra[8], rb[8];
    MkLane<TU> ua, ub;
    fetch_w2(tile, ra);
    fetch_u(tile, ua);
    // keeps the second tile's loads behind the first's, so that the first
    // tile's waits leave them in flight
    asm volatile("" ::: "memory");
    fetch_w2(tile + G, rb);
    fetch_u(tile + G, ub);
    // buffer 0 holds the tiles of set a, buffer 1 those of set b; a buffer
    // is written again only after the barrier that follows its last reader
#pragma unroll
    for (int it = 0; it < kMkPipeTiles; ++it) {
        if (tile >= tend) break;
        if (it & 1) {
            stage(1, rb);
            __syncthreads();
            fetch_w2(tile + 2 * G, rb);
            product(1, tile, ub);
            fetch_u(tile + 2 * G, ub);
        } else {
            stage(0, ra);
            __syncthreads();
            fetch_w2(tile + 2 * G, ra);
            product(0, tile, ua);
            fetch_u(tile + 2 * G, ua);
        }
        tile += G;
    }
}

// Tile mass relative to the row maximum M: sum over the tile of 2^((l - M) s).
__device__ __forceinline__ double mk_tile_mass(float2 st, float M, float s) {
    return st.x > -__builtin_inff()
               ? (double)st.y * (double)__builtin_amdgcn_exp2f((st.x - M) * s)
               : 0.0;
}

// One workgroup per request; thread i owns the run of tiles [i tp, (i + 1) tp)
// and keeps its statistics in registers (NB >= tp, else batches of NB).
//  1. every load of the request is issued at once: its parameters and the
//     statistics of every run.  Each wave reduces its threads' NaN flags and
//     maxima (argmax at T = 0), and the four wave results meet in shared
//     memory: the row maximum M;
//  2. each thread's run mass relative to M, an inclusive scan per wave and
//     the wave totals in shared memory give every thread its exclusive
//     prefix; the first thread (in thread order) whose run holds u * total
//     is found by a ballot per wave and the first wave with a hit;
//  3. the hit thread walks its run in registers: the tile and the target
//     left inside it;
//  4. the first wave reads that tile's 64 logits (one per lane) and a wave
//     scan finds the token.
// Four barriers in all.  The CDF must exceed the target strictly; a target at
// or past the total, which only rounding can produce, takes the last tile
// and token of positive mass.  Lane indices in the first wave come from
// ballots, so they are wave-uniform and neighbouring prefixes are read with
// readlane.
template <int NB>
__global__ void __launch_bounds__(kBlock) markov_sample_kernel(MarkovArgs a) {
    __shared__ float s_wf[kWaves];
    __shared__ int s_wi[kWaves], s_wb[kWaves], s_wl[kWaves], s_wh[kWaves];
    __shared__ double s_wd[kWaves];
    __shared__ int s_tile;
    __shared__ double s_tin;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x;
    const int k = a.k;
    const int V = a.V;
    const int nt = a.ntiles;
    const int tp = (nt + kBlock - 1) / kBlock;  // tiles per thread
    const int nb = (tp + NB - 1) / NB;          // register batches per run
    const int t0 = tid * tp;
    const float2 *ts = a.tstats + (size_t)r * nt;
    float2 st[NB];
    auto load_batch = [&](int b) {
#pragma unroll
        for (int i = 0; i < NB; ++i) st[i] = ts[min(t0 + b * NB + i, nt - 1)];
    };
    auto valid = [&](int b, int i) { return b * NB + i < tp && t0 + b * NB + i < nt; };
    const float T = a.temp[r];
    const int32_t anc = a.anchor[r];
    // the request's flag from the earlier steps (none before step 1)
    const uint32_t rbad = k > 1 ? a.bad[r] : 0u;
    const float u = a.ud[(size_t)r * a.gamma + (k - 1)];
    load_batch(0);
    bool ok = mk_temperature_ok(T) && anc >= 0 && anc < V && rbad == 0u;
    if (T != 0.0f && !(u >= 0.0f && u < 1.0f)) ok = false;
    const float s = (T > 0.0f && ok) ? (float)(kLog2e / (double)T) : 1.0f;
    int token = -1;

    // pass 1: run maximum, NaN flags, greedy argmax; wave results, then the
    // block's from the four waves
    float lm = -__builtin_inff();
    int bad = 0;
    int bi = 0x7fffffff;
    for (int b = 0; b < nb; ++b) {
        if (b > 0) load_batch(b);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (!valid(b, i)) continue;
            const float2 x = st[i];
            if (x.x != x.x || (T != 0.0f && x.y != x.y)) bad = 1;
            if (T == 0.0f)
                argmax_combine(lm, bi, x.x, __float_as_int(x.y));
            else
                lm = fmaxf(lm, x.x);
        }
    }
    bad = wave_max_i(bad);
    if (T == 0.0f)
        wave_argmax(lm, bi);
    else
        lm = wave_max(lm);
    if (lane == 0) {
        s_wf[wave] = lm;
        s_wi[wave] = bi;
        s_wb[wave] = bad;
    }
    __syncthreads();
    float M = s_wf[0];
    int B = s_wi[0];
    bad = s_wb[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        bad = max(bad, s_wb[w]);
        if (T == 0.0f)
            argmax_combine(M, B, s_wf[w], s_wi[w]);
        else
            M = fmaxf(M, s_wf[w]);
    }
    if (ok && T == 0.0f) {
        ok = !bad && M < __builtin_inff() && B != 0x7fffffff;
        token = B;
    } else if (ok) {
        ok = !bad && M > -__builtin_inff() && M < __builtin_inff();
        if (ok) {
            // pass 2: run masses relative to M, the exclusive prefix of every
            // run, the run holding u * W
            double lsum = 0.0;
            int lastp = -1;
            for (int b = 0; b < nb; ++b) {
                if (nb > 1) load_batch(b);
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    if (!valid(b, i)) continue;
                    const double w = mk_tile_mass(st[i], M, s);
                    lsum += w;
                    if (w > 0.0) lastp = t0 + b * NB + i;
                }
            }
            const double incl = wave_incl_scan_dpp(lsum);
            double excl = __shfl_up(incl, 1, 64);
            if (lane == 0) excl = 0.0;
            const int wlast = wave_max_i(lastp);
            if (lane == 63) s_wd[wave] = incl;
            if (lane == 0) s_wl[wave] = wlast;
            __syncthreads();
            double base = 0.0, W = 0.0;
            int last = -1;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                if (w < wave) base += s_wd[w];
                W += s_wd[w];
                last = max(last, s_wl[w]);
            }
            excl += base;
            const double tt = (double)u * W;
            const uint64_t hm = __ballot(lsum > 0.0 && excl + lsum > tt);
            if (lane == 0) s_wh[wave] = hm ? __builtin_ctzll(hm) : 64;
            __syncthreads();
            int hw = -1;
#pragma unroll
            for (int w = kWaves - 1; w >= 0; --w)
                if (s_wh[w] < 64) hw = w;
            if (hw < 0) {  // u * W at or past the total (rounding)
                if (tid == 0) {
                    s_tile = last;
                    s_tin = INFINITY;
                }
            } else if (wave == hw && lane == s_wh[hw]) {
                // pass 3: the hit thread walks its run
                double run = excl;
                int tl = -1;
                double tin = INFINITY;
                for (int b = 0; b < nb && tl < 0; ++b) {
                    if (nb > 1) load_batch(b);
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        if (!valid(b, i) || tl >= 0) continue;
                        const double w = mk_tile_mass(st[i], M, s);
                        if (w > 0.0 && run + w > tt) {
                            tl = t0 + b * NB + i;
                            tin = tt - run;
                        }
                        run += w;
                    }
                }
                if (tl < 0) tl = lastp;  // rounding inside the run: its last tile with mass
                s_tile = tl;
                s_tin = tin;
            }
            __syncthreads();
            int tile = s_tile;
            const double tin = s_tin;
            if (tile < 0) tile = 0;  // unreachable: the tile holding M has mass
            if (tid < 64) {
                // the tile's logits, one per lane, in id order
                const float m = ts[tile].x;
                const long v = (long)tile * kMkTile + lane;
                const float *lrow = a.out_logits + ((long)r * a.gamma + (k - 1)) * V;
                const float e = (v < V && m > -__builtin_inff())
                                    ? __builtin_amdgcn_exp2f((lrow[min(v, (long)V - 1)] - m) * s)
                                    : 0.0f;
                const double w3 = (double)e * (double)__builtin_amdgcn_exp2f((m - M) * s);
                const double inc3 = wave_incl_scan_dpp(w3);
                const uint64_t h3 = __ballot(w3 > 0.0 && inc3 > tin);
                const uint64_t pos3 = __ballot(w3 > 0.0);
                if (h3)
                    token = tile * kMkTile + __builtin_ctzll(h3);
                else
                    token = pos3 ? tile * kMkTile + 63 - __builtin_clzll(pos3) : -1;
            }
            ok = token >= 0;
        }
    }
    if (tid == 0) {
        const uint32_t nbad = (rbad || !ok) ? 1u : 0u;
        a.bad[r] = nbad;
        a.out_tok[(size_t)r * a.gamma + (k - 1)] = ok ? token : -1;
        if (k == a.gamma && nbad) {
            for (int q = 0; q < a.gamma; ++q) a.out_tok[(size_t)r * a.gamma + q] = -1;
            atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
        }
    }
}

// fp32 value of x rounded to bf16 (nearest, ties to even; finite x).
__device__ __forceinline__ float bf16_round(float x) {
    const uint32_t b = __float_as_uint(x);
    return __uint_as_float((b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u);
}

// ---------------------------------------------------------------------------
// RNN serial head: the gated state update of step k
// ---------------------------------------------------------------------------

constexpr int kRnnReq = 4;      // requests per workgroup of the gate product
constexpr int kRnnKS = 32;      // workgroups splitting the 2 rank + hidden rows
constexpr int kRnnRowsPerWave = (2 * kMkRank + SPEC_RNN_MAX_HIDDEN + 4 * kRnnKS - 1) / (4 * kRnnKS);
constexpr int kRnnMaxHidden = SPEC_RNN_MAX_HIDDEN;
constexpr int kRnnCols = 2 * kMkRank;  // update-gate and candidate columns

struct RnnArgs {
    const uint16_t *W1;     // [V][rank] bf16 embedding
    const float *H;         // [R][gamma][hidden] backbone hidden states
    const uint16_t *Wg;     // [2 rank + hidden][2 rank] bf16: update-gate | candidate columns
    const float *bg;        // [2 rank]
    const int32_t *anchor;  // [R]
    const int32_t *tok;     // [R][gamma] drafted tokens (the previous step's)
    const float *s_prev;    // [R][rank]
    float *s_next;          // [R][rank]
    float *part;            // [kRnnKS][R][2 rank] partial gate sums
    uint16_t *bsplit;       // [3][R][rank] bf16 parts of s_next
    float *out_state;       // [R][gamma][rank] or null
    int R, gamma, V, hidden, k;
};

// Element e of request r's concatenation c = [s_{k-1}; W1[x_{k-1}]; h_k].
__device__ __forceinline__ float rnn_c(const RnnArgs &a, int r, int e) {
    if (e < kMkRank) return a.k > 1 ? a.s_prev[(size_t)r * kMkRank + e] : 0.0f;
    if (e < 2 * kMkRank) {
        const int x = a.k == 1 ? a.anchor[r] : a.tok[(size_t)r * a.gamma + (a.k - 2)];
        return (x >= 0 && x < a.V)
                   ? __uint_as_float((uint32_t)a.W1[(size_t)x * kMkRank + (e - kMkRank)] << 16)
                   : 0.0f;
    }
    return a.H[((size_t)r * a.gamma + (a.k - 1)) * a.hidden + (e - 2 * kMkRank)];
}

// Partial gate products: workgroup (request block q0, row block kb) takes
// rows [kb rpb, (kb + 1) rpb) of c Wg for 4 requests, one quarter per wave;
// lane l keeps columns 8 l .. 8 l + 7 for the 4 requests, each Wg row read
// as one 1 KB wave load.  The waves' sums are added in LDS in wave order and
// written to part[kb].
__global__ void __launch_bounds__(kBlock) rnn_gate_kernel(RnnArgs a) {
    __shared__ float cv[kRnnReq][4 * kRnnRowsPerWave];
    __shared__ float red[4][kRnnReq][kRnnCols];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int dc = 2 * kMkRank + a.hidden;
    const int rpb = (dc + kRnnKS - 1) / kRnnKS;  // rows per workgroup (<= 4 kRnnRowsPerWave)
    const int q0 = blockIdx.x * kRnnReq, kb = blockIdx.y;
    const int i0 = kb * rpb;
    for (int t = tid; t < kRnnReq * rpb; t += kBlock) {
        const int q = t / rpb, e = i0 + (t - q * rpb);
        cv[q][t - q * rpb] = (q0 + q < a.R && e < dc) ? rnn_c(a, q0 + q, e) : 0.0f;
    }
    __syncthreads();
    const int rpw = (rpb + 3) / 4;
    const int w0 = wave * rpw;
    float acc[kRnnReq][8];
#pragma unroll
    for (int q = 0; q < kRnnReq; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[q][j] = 0.0f;
#pragma unroll
    for (int t = 0; t < kRnnRowsPerWave; ++t) {
        const int ir = w0 + t;             // row within the workgroup's block
        const int i = i0 + ir;
        const bool in = t < rpw && ir < rpb && i < dc;
        const uint4 wv = *reinterpret_cast<const uint4 *>(a.Wg + (size_t)(in ? i : 0) * kRnnCols +
                                                          lane * 8);
        const float w[8] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y),
                            bf16_lo(wv.z), bf16_hi(wv.z), bf16_lo(wv.w), bf16_hi(wv.w)};
        if (in) {
#pragma unroll
            for (int q = 0; q < kRnnReq; ++q) {
                const float cq = cv[q][ir];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[q][j] = fmaf(cq, w[j], acc[q][j]);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kRnnReq; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) red[wave][q][lane * 8 + j] = acc[q][j];
    __syncthreads();
    for (int t = tid; t < kRnnReq * kRnnCols; t += kBlock) {
        const int q = t / kRnnCols, col = t - q * kRnnCols;
        if (q0 + q < a.R) {
            const float v = ((red[0][q][col] + red[1][q][col]) + red[2][q][col]) + red[3][q][col];
            a.part[((size_t)kb * a.R + q0 + q) * kRnnCols + col] = v;
        }
    }
}

// The update of unit u of request r: the partial sums added in row-block
// order, z = sigmoid, n = tanh, s_k = (1 - z) s_{k-1} + z n, and its three bf16
// parts (hi = bf16(s), mid = bf16(s - hi), lo = bf16(s - hi - mid); both
// differences are exact in fp32).
__global__ void __launch_bounds__(kBlock) rnn_state_kernel(RnnArgs a) {
    const int t = blockIdx.x * kBlock + threadIdx.x;
    if (t >= a.R * kMkRank) return;
    const int r = t / kMkRank, u = t - r * kMkRank;
    float gz = a.bg[u], gn = a.bg[kMkRank + u];
    for (int kb = 0; kb < kRnnKS; ++kb) {
        const float *pp = a.part + ((size_t)kb * a.R + r) * kRnnCols;
        gz += pp[u];
        gn += pp[kMkRank + u];
    }
    const float z = 1.0f / (1.0f + expf(-gz));
    const float n = tanhf(gn);
    const float sp = a.k > 1 ? a.s_prev[t] : 0.0f;
    const float sn = (1.0f - z) * sp + z * n;
    a.s_next[t] = sn;
    if (a.out_state) a.out_state[((size_t)r * a.gamma + (a.k - 1)) * kMkRank + u] = sn;
    const float hi = bf16_round(sn);
    const float mid = bf16_round(sn - hi);
    const float lo = bf16_round(sn - hi - mid);
    const size_t plane = (size_t)a.R * kMkRank;
    a.bsplit[t] = (uint16_t)(__float_as_uint(hi) >> 16);
    a.bsplit[plane + t] = (uint16_t)(__float_as_uint(mid) >> 16);
    a.bsplit[2 * plane + t] = (uint16_t)(__float_as_uint(lo) >> 16);
}


namespace {

size_t mk_round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device, cached per device (0 if unknown).
constexpr int kMkMaxDevices = 64;
std::atomic<int> g_mk_cus[kMkMaxDevices];
int mk_device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMkMaxDevices) return 0;
    int c = g_mk_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    g_mk_cus[dev].store(c, std::memory_order_relaxed);
    return c;
}

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

// Step k's logits (U_k + B W2 with the B rows of NSPLIT) and draw.
template <int NSPLIT>
void mk_launch_step(MarkovArgs a, const MkPlan &p, bool bf, hipStream_t st) {
    const int R = a.R, V = a.V;
    // whole tiles in 16-byte aligned rows take the vector kernel; the ragged
    // last tile (or every tile of an odd V or unaligned rows) the guarded one
    const int nfull = (V % 8 == 0 && a.vec) ? V / kMkTile : 0;
    const int tp = (p.ntiles + kBlock - 1) / kBlock;  // tiles per thread of the sampling block
    // persistent: wide tiles of 128 ids, one workgroup of 512 threads per CU
    // (the odd 64-id tile, if any, goes to the per-tile launch below)
    // SPECMARKOV_TILES=1 in the environment keeps the per-tile launches (for
    // comparisons)
    constexpr int kH = 2;
    const char *pt = getenv("SPECMARKOV_TILES");
    const bool per_tile = pt && pt[0] == '1';
    const int cus = NSPLIT == 1 && R == kMkRows && nfull >= kH && !per_tile ? mk_device_cus() : 0;
    const int nwide = nfull / kH;
    const int g = nwide < cus ? nwide : cus;
    int done = 0;
    if (g > 0 && (nwide + g - 1) / g <= kMkPipeTiles) {
        const size_t lds = 2 * sizeof(uint16_t) * kMkTile * kH * kMkLdsStride;
        static std::atomic<int> attr{0};
        bool ok = attr.load(std::memory_order_relaxed) != 0;
        if (!ok) {
            ok = hipFuncSetAttribute(
                     reinterpret_cast<const void *>(&markov_logits_pipe_kernel<uint16_t, kH>),
                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess &&
                 hipFuncSetAttribute(
                     reinterpret_cast<const void *>(&markov_logits_pipe_kernel<float, kH>),
                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
            if (ok) attr.store(1, std::memory_order_relaxed);
        }
        if (ok) {
            a.tile0 = 0;
            a.tile1 = nwide;
            if (bf)
                hipLaunchKernelGGL((markov_logits_pipe_kernel<uint16_t, kH>), dim3(g),
                                   dim3(kBlock * kH), lds, st, a);
            else
                hipLaunchKernelGGL((markov_logits_pipe_kernel<float, kH>), dim3(g),
                                   dim3(kBlock * kH), lds, st, a);
            done = nwide * kH;
        }
    }
    if (done > 0) {
        if (done < nfull) {
            a.tile0 = done;
            if (bf)
                hipLaunchKernelGGL((markov_logits_kernel<uint16_t, true, NSPLIT>),
                                   dim3(nfull - done), dim3(kBlock), 0, st, a);
            else
                hipLaunchKernelGGL((markov_logits_kernel<float, true, NSPLIT>),
                                   dim3(nfull - done), dim3(kBlock), 0, st, a);
        }
    } else if (nfull > 0) {
        a.tile0 = 0;
        if (bf)
            hipLaunchKernelGGL((markov_logits_kernel<uint16_t, true, NSPLIT>), dim3(nfull),
                               dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL((markov_logits_kernel<float, true, NSPLIT>), dim3(nfull),
                               dim3(kBlock), 0, st, a);
    }
    if (nfull < p.ntiles) {
        a.tile0 = nfull;
        if (bf)
            hipLaunchKernelGGL((markov_logits_kernel<uint16_t, false, NSPLIT>),
                               dim3(p.ntiles - nfull), dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL((markov_logits_kernel<float, false, NSPLIT>),
                               dim3(p.ntiles - nfull), dim3(kBlock), 0, st, a);
    }
    if (tp <= 8)
        hipLaunchKernelGGL(markov_sample_kernel<8>, dim3(R), dim3(kBlock), 0, st, a);
    else
        hipLaunchKernelGGL(markov_sample_kernel<16>, dim3(R), dim3(kBlock), 0, st, a);
}

// Workspace of the RNN head: the Markov head's, then two fp32 states and the
// three bf16 parts of the current one.
struct RnnPlan {
    MkPlan mk;
    size_t off_s0, off_s1, off_split, off_part, bytes;
};

bool rnn_plan(long R, long V, RnnPlan &p) {
    mk_plan(R, V, p.mk);
    const size_t sb = sizeof(float) * (size_t)R * kMkRank;
    p.off_s0 = p.mk.bytes;
    p.off_s1 = mk_round_up(p.off_s0 + sb, 256);
    p.off_split = mk_round_up(p.off_s1 + sb, 256);
    p.off_part = mk_round_up(p.off_split + 3 * sizeof(uint16_t) * (size_t)R * kMkRank, 256);
    p.bytes = mk_round_up(p.off_part + sizeof(float) * kRnnKS * (size_t)R * kRnnCols, 256);
    return true;
}

// Shared argument set-up of the two draft heads.
int mk_setup(const void *U, int u_dtype, const void *W1, const void *W2, int w_dtype,
             const int32_t *anchor, const float *temperature, const float *u_draft, int R,
             int gamma, int V, int rank, int32_t *out_tok, float *out_logits, void *workspace,
             const MkPlan &p, MarkovArgs &a) {
    char *ws = (char *)workspace;
    a = MarkovArgs{};
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
    a.out_tok = out_tok;
    a.out_logits = out_logits;
    a.tstats = (float2 *)(ws + p.off_stats);
    a.bad = (uint32_t *)(ws + p.off_bad);
    a.ctl = (Control *)ws;
    const size_t ub = (u_dtype == SPEC_BF16) ? 2 : 4;
    a.vec = (V % 4 == 0) && ((uintptr_t)U % (4 * ub) == 0) && ((uintptr_t)out_logits % 16 == 0);
    (void)W2; (void)w_dtype; (void)rank; (void)anchor; (void)temperature; (void)u_draft;
    return SPEC_OK;
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
    MarkovArgs a;
    mk_setup(U, u_dtype, W1, W2, w_dtype, anchor, temperature, u_draft, R, gamma, V, rank,
             out_draft_tokens, out_draft_logits, workspace, p, a);
    hipStream_t st = (hipStream_t)stream;
    for (int k = 1; k <= gamma; ++k) {
        a.k = k;
        mk_launch_step<1>(a, p, u_dtype == SPEC_BF16, st);
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

size_t spec_rnn_workspace_bytes(int R, int gamma, int V, int rank, int hidden) {
    if (R < 0 || gamma < 0 || V < 1 || V > SPEC_MAX_VOCAB || rank != kMkRank || hidden < 1 ||
        hidden > kRnnMaxHidden)
        return 0;
    RnnPlan p;
    rnn_plan(R > 0 ? R : 1, V, p);
    return p.bytes;
}

int spec_rnn_draft_sample(const void *U, int u_dtype, const void *W1, const void *W2, int w_dtype,
                          const float *hidden_states, int hidden, const void *Wg, const float *bg,
                          const int32_t *anchor, const float *temperature, const float *u_draft,
                          int R, int gamma, int V, int rank, int32_t *out_draft_tokens,
                          float *out_draft_logits, float *out_state, void *workspace,
                          size_t workspace_bytes, void *stream) {
    if (R < 0 || gamma < 0 || V < 1 || hidden < 1) return SPEC_EINVAL;
    if ((u_dtype != SPEC_F32 && u_dtype != SPEC_BF16) || w_dtype != SPEC_BF16) return SPEC_EDTYPE;
    if (rank != kMkRank || V > SPEC_MAX_VOCAB || hidden > kRnnMaxHidden) return SPEC_EUNSUPPORTED;
    if (R == 0 || gamma == 0) return SPEC_OK;
    if (!U || !W1 || !W2 || !hidden_states || !Wg || !bg || !anchor || !temperature || !u_draft ||
        !out_draft_tokens || !out_draft_logits)
        return SPEC_EINVAL;
    if (((uintptr_t)W1 & 15u) || ((uintptr_t)W2 & 15u) || ((uintptr_t)Wg & 15u)) return SPEC_EINVAL;
    RnnPlan p;
    rnn_plan(R, V, p);
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < p.bytes)
        return SPEC_EWORKSPACE;
    char *ws = (char *)workspace;
    MarkovArgs a;
    mk_setup(U, u_dtype, W1, W2, w_dtype, anchor, temperature, u_draft, R, gamma, V, rank,
             out_draft_tokens, out_draft_logits, workspace, p.mk, a);
    a.bsplit = (const uint16_t *)(ws + p.off_split);
    RnnArgs g{};
    g.W1 = (const uint16_t *)W1;
    g.H = hidden_states;
    g.Wg = (const uint16_t *)Wg;
    g.bg = bg;
    g.anchor = anchor;
    g.tok = out_draft_tokens;
    g.bsplit = (uint16_t *)(ws + p.off_split);
    g.part = (float *)(ws + p.off_part);
    g.out_state = out_state;
    g.R = R;
    g.gamma = gamma;
    g.V = V;
    g.hidden = hidden;
    float *s0 = (float *)(ws + p.off_s0), *s1 = (float *)(ws + p.off_s1);
    hipStream_t st = (hipStream_t)stream;
    const dim3 ggrid((R + kRnnReq - 1) / kRnnReq, kRnnKS);
    const dim3 sgrid((R * kMkRank + kBlock - 1) / kBlock);
    for (int k = 1; k <= gamma; ++k) {
        g.k = k;
        g.s_prev = (k & 1) ? s0 : s1;  // unread at k = 1 (s_0 = 0)
        g.s_next = (k & 1) ? s1 : s0;
        hipLaunchKernelGGL(rnn_gate_kernel, ggrid, dim3(kBlock), 0, st, g);
        hipLaunchKernelGGL(rnn_state_kernel, sgrid, dim3(kBlock), 0, st, g);
        a.k = k;
        mk_launch_step<3>(a, p.mk, u_dtype == SPEC_BF16, st);
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
