// common.h -- device helpers shared by the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kBlock = 256;               // threads per workgroup (4 wave64s)
constexpr int kWaves = kBlock / 64;
constexpr int kMaxGamma = 64;             // largest draft length (gamma) accepted
constexpr uint32_t kSpinLimit = 1u << 20; // polls before a cross-wave wait gives up
constexpr int kMaxChunks = 4096;          // chunks per row
constexpr double kLog2e = 1.4426950408889634;
constexpr double kLn2 = 0.6931471805599453;

// Workspace control block (offset 0, 256 bytes).
struct Control {
    uint32_t tag_next;   // the next verification call's launch tag (0 after init)
    uint32_t status;     // SPEC_DEV_* bits
    uint32_t tag_call;   // the running verification call's launch tag
    uint32_t pad[61];
};
static_assert(sizeof(Control) == 256, "control block size");

__device__ __forceinline__ uint32_t atomic_load_u32(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_u32(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_or_u32(uint32_t *p, uint32_t v) {
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> struct EltBytes;
template <> struct EltBytes<float> { static constexpr int value = 4; };
template <> struct EltBytes<uint16_t> { static constexpr int value = 2; };

// Loads EPV consecutive logits starting at element e of `row` (e a multiple of
// EPV; EPV * sizeof(T) <= 16) as fp32.
template <typename T, int EPV> struct VecLoad;

template <int EPV> struct VecLoad<float, EPV> {
    __device__ __forceinline__ static void run(const float *row, long e, float *out) {
        if constexpr (EPV == 4) {
            float4 v = *reinterpret_cast<const float4 *>(row + e);
            out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
        } else if constexpr (EPV == 2) {
            float2 v = *reinterpret_cast<const float2 *>(row + e);
            out[0] = v.x; out[1] = v.y;
        } else {
            static_assert(EPV == 1, "fp32 vector width");
            out[0] = row[e];
        }
    }
};

template <int EPV> struct VecLoad<uint16_t, EPV> {
    __device__ __forceinline__ static void run(const uint16_t *row, long e, float *out) {
        if constexpr (EPV == 8) {
            uint4 v = *reinterpret_cast<const uint4 *>(row + e);
            out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
            out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
            out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
            out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
        } else if constexpr (EPV == 4) {
            uint2 v = *reinterpret_cast<const uint2 *>(row + e);
            out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
            out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
        } else if constexpr (EPV == 2) {
            uint32_t v = *reinterpret_cast<const uint32_t *>(row + e);
            out[0] = bf16_lo(v); out[1] = bf16_hi(v);
        } else {
            static_assert(EPV == 1, "bf16 vector width");
            out[0] = __uint_as_float(((uint32_t)row[e]) << 16);
        }
    }
};

template <typename T>
__device__ __forceinline__ float load_one(const T *row, long e) {
    float v;
    VecLoad<T, 1>::run(row, e, &v);
    return v;
}

// ---------------------------------------------------------------------------
// wave / block reductions (fixed association order: every lane and every
// workgroup running the same code on the same values gets the same bits)
// ---------------------------------------------------------------------------

// Wave-wide reductions with every one of the 64 lanes active.  Four DPP
// steps inside each row of 16 lanes (swap neighbours, swap pairs, mirror the
// half-row, mirror the row) leave every lane of a row holding that row's
// result; the four row results are read into scalar registers and combined,
// so the value returned is uniform across the wave.  DPP moves run in the
// VALU pipeline: no LDS round trip per step, unlike ds_bpermute shuffles.
constexpr int kDppSwap1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15 - i within 16

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = dpp_i<CTRL>((int)(b & 0xffffffffLL));
    const int hi = dpp_i<CTRL>((int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    const long long b = __double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(b & 0xffffffffLL), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | lo);
}

// wave_max propagates NaN (IEEE maximum, one v_maximum3 per step); callers
// pass lane maxima built with fmaxf, which are never NaN.
__device__ __forceinline__ float wave_max(float v) {
    v = __builtin_elementwise_maximum(v, dpp_f<kDppSwap1>(v));
    v = __builtin_elementwise_maximum(v, dpp_f<kDppSwap2>(v));
    v = __builtin_elementwise_maximum(v, dpp_f<kDppHalfMirror>(v));
    v = __builtin_elementwise_maximum(v, dpp_f<kDppMirror>(v));
    return __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(readlane_f(v, 0), readlane_f(v, 16)),
        __builtin_elementwise_maximum(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_d<kDppSwap1>(v);
    v += dpp_d<kDppSwap2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}
__device__ __forceinline__ float wave_sum_f(float v) {
    v += dpp_f<kDppSwap1>(v);
    v += dpp_f<kDppSwap2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ int wave_max_i(int v) {
    v = max(v, dpp_i<kDppSwap1>(v));
    v = max(v, dpp_i<kDppSwap2>(v));
    v = max(v, dpp_i<kDppHalfMirror>(v));
    v = max(v, dpp_i<kDppMirror>(v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_min_i(int v) {
    v = min(v, dpp_i<kDppSwap1>(v));
    v = min(v, dpp_i<kDppSwap2>(v));
    v = min(v, dpp_i<kDppHalfMirror>(v));
    v = min(v, dpp_i<kDppMirror>(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// Wave inclusive prefix sums in lane order with DPP moves only: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16 (lanes whose source lies before
// the row start read 0), then lane 15's sum added to rows 1 and 3 and lane
// 31's to rows 2 and 3.  No LDS round trip per step, unlike the
// ds_bpermute shuffles of wave_incl_scan.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// DPP move in which lanes of rows outside ROW_MASK, and lanes whose source
// is out of range, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp0_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp0_d(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = dpp0_i<CTRL, ROW_MASK>((int)(b & 0xffffffffLL));
    const int hi = dpp0_i<CTRL, ROW_MASK>((int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double wave_incl_scan_dpp(double v) {
    v += dpp0_d<kDppRowShr1, 0xf>(v);
    v += dpp0_d<kDppRowShr2, 0xf>(v);
    v += dpp0_d<kDppRowShr4, 0xf>(v);
    v += dpp0_d<kDppRowShr8, 0xf>(v);
    v += dpp0_d<kDppRowBcast15, 0xa>(v);
    v += dpp0_d<kDppRowBcast31, 0xc>(v);
    return v;
}
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
    v += (uint32_t)dpp0_i<kDppRowShr1, 0xf>((int)v);
    v += (uint32_t)dpp0_i<kDppRowShr2, 0xf>((int)v);
    v += (uint32_t)dpp0_i<kDppRowShr4, 0xf>((int)v);
    v += (uint32_t)dpp0_i<kDppRowShr8, 0xf>((int)v);
    v += (uint32_t)dpp0_i<kDppRowBcast15, 0xa>((int)v);
    v += (uint32_t)dpp0_i<kDppRowBcast31, 0xc>((int)v);
    return v;
}

// Lane l's value and that of lane l ^ P (P = 16 or 32) with the gfx950
// permlane swaps: lo = the value of the pair's lane in the lower row (P = 16)
// or half (P = 32), hi = that of the upper one, the same pair in both lanes,
// so that both lanes combine the two values in the same order.  No LDS round
// trip, unlike a ds_bpermute shuffle.
template <int P>
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t &lo, uint32_t &hi) {
    static_assert(P == 16 || P == 32, "row or half partner");
    if constexpr (P == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        lo = r[0];
        hi = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        lo = r[0];
        hi = r[1];
    }
}

// Wave inclusive prefix sum (fp64) in lane order.
__device__ __forceinline__ double wave_incl_scan(double v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double n = __shfl_up(v, o, 64);
        if ((int)(threadIdx.x & 63) >= o) v += n;
    }
    return v;
}
// (value, index): larger value wins, equal values -> smaller index.
__device__ __forceinline__ void argmax_combine(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float &v, int &i) {
    const float v2 = dpp_f<CTRL>(v);
    const int i2 = dpp_i<CTRL>(i);
    argmax_combine(v, i, v2, i2);
}
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
    argmax_step<kDppSwap1>(v, i);
    argmax_step<kDppSwap2>(v, i);
    argmax_step<kDppHalfMirror>(v, i);
    argmax_step<kDppMirror>(v, i);
    float bv = readlane_f(v, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int l = 16; l < 64; l += 16)
        argmax_combine(bv, bi, readlane_f(v, l), __builtin_amdgcn_readlane(i, l));
    v = bv;
    i = bi;
}

}  // namespace sv
