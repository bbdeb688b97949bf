// tree.hip -- greedy (T = 0) verification of draft trees on gfx950.
//
// Method: a speculative-decoding survey (zhifeiding.github.io), sec. 2.3: a
// tree draft expands several branches per node and the target scores the
// whole tree in one pass; the DART reading note (zhongzhuzhou.org), sec. 2.3:
// at temperature zero the verifier follows the target's argmax along the
// candidate paths (the pages give no T > 0 rule, so none is offered here).
// Node v (parent p(v) < v, draft token x_v) is accepted when its parent is
// and x_v is the argmax of the target row of p(v) (lowest id on ties); the
// walk goes to the accepted child (the lowest-index one among equal
// siblings) and stops at a node with none, whose row's argmax is the bonus
// or correction token.
//
// Only the rows on the accepted path are needed.  Level l of the walk reads
// the row of node c_l (c_0 = the root); launch l of max_depth + 2:
//  * every workgroup of request r first takes the step from level l - 1: the
//    argmax g of row c_{l-1} (one 64-bit word, see below), then the child of
//    c_{l-1} carrying g found with a wave ballot; all workgroups of the
//    request compute the same c_l, and slice 0's writes it and the outputs
//    (or ends the walk: no such child, g is the bonus token);
//  * then workgroup (slice s, request r) takes logits [s L, (s + 1) L) of
//    row c_l with 16-byte loads, reduces them to (value, id) and merges that
//    into the level's word with one atomicMax: the word holds the value's
//    order-preserving bits above the complement of the id, so the largest
//    word is the row's maximum at its lowest id, whatever the order of the
//    merges.  A NaN or +-inf logit sets the level's fault flag.
// No workgroup waits for another: each level's word is complete when the
// next launch starts.  tree_init_kernel checks the trees first (parents in
// [0, v), tokens in [0, V), 1 <= n <= M, depth <= max_depth) and clears the
// words and the outputs.
#include <math.h>

#include "common.h"

namespace sv {

constexpr int kTreeMaxNodes = SPEC_TREE_MAX_NODES;

constexpr int kTreeSlice = 8192;  // logits per workgroup and row

struct TreeArgs {
    const void *logits;      // [R][M][V]
    const int32_t *parent;   // [R][M]
    const int32_t *tokens;   // [R][M]
    const int32_t *n_nodes;  // [R]
    int R, M, V, S, max_depth, level;
    int32_t *out_acc;        // [R] accepted draft nodes (-1: invalid request)
    int32_t *out_path;       // [R][M] accepted node indices, -1 padded
    int32_t *out_tok;        // [R][M] path tokens then the bonus, -1 padded
    int32_t *node;           // [R][L] c_l, the node level l reads (-1: walk over)
    uint64_t *key;           // [R][L] level l's argmax word
    uint32_t *fault;         // [R][L] level l's row held a NaN or +-inf
    int L;                   // levels stored per request (max_depth + 1)
    Control *ctl;
};

// Order-preserving bits of a finite float (larger float, larger word).
__device__ __forceinline__ uint32_t tree_ord(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ void __launch_bounds__(64) tree_init_kernel(TreeArgs a) {
    __shared__ int dep[kTreeMaxNodes];
    const int r = blockIdx.x, lane = threadIdx.x;
    const size_t rb = (size_t)r * a.M;
    const int n = a.n_nodes[r];
    bool ok = n >= 1 && n <= a.M;
    const int nn = ok ? n : 0;
    for (int v = 1 + lane; v < nn; v += 64) {
        const int p = a.parent[rb + v];
        const int x = a.tokens[rb + v];
        ok = ok && p >= 0 && p < v && x >= 0 && x < a.V;
        dep[v] = p;  // parents first, depths below
    }
    ok = __syncthreads_and(ok);
    if (ok && lane == 0) {
        // depths in index order (every parent comes before its children)
        int dmax = 0;
        dep[0] = 0;
        for (int v = 1; v < nn; ++v) {
            const int d = dep[dep[v]] + 1;
            dep[v] = d;
            dmax = d > dmax ? d : dmax;
        }
        dep[0] = dmax;
    }
    __syncthreads();
    if (ok) ok = dep[0] <= a.max_depth;
    for (int v = lane; v < a.M; v += 64) {
        a.out_path[rb + v] = -1;
        a.out_tok[rb + v] = -1;
    }
    for (int l = lane; l < a.L; l += 64) {
        a.key[(size_t)r * a.L + l] = 0ull;
        a.fault[(size_t)r * a.L + l] = 0u;
        a.node[(size_t)r * a.L + l] = (l == 0 && ok) ? 0 : -1;
    }
    if (lane == 0) {
        a.out_acc[r] = -1;
        if (!ok) atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
    }
}

// Argmax of one logit into (v, i), lowest id on ties; a NaN or +-inf marks bad.
__device__ __forceinline__ void tree_take(float z, int id, float &v, int &i, int &bad) {
    if (z - z != 0.0f) bad = 1;
    if (z > v || (z == v && id < i)) {
        v = z;
        i = id;
    }
}

template <typename T, int EPV>
__global__ void __launch_bounds__(kBlock) tree_level_kernel(TreeArgs a) {
    __shared__ float wv[kWaves];
    __shared__ int wi[kWaves], wb[kWaves];
    __shared__ int cur_s;
    const int r = blockIdx.y, s = blockIdx.x, l = a.level;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t rb = (size_t)r * a.M, lb = (size_t)r * a.L;
    int cur;
    if (l == 0) {
        cur = a.node[lb];
    } else {
        // the step from level l - 1 (wave 0; every workgroup alike)
        const int prev = a.node[lb + l - 1];
        if (prev < 0) return;
        if (wave == 0) {
            const uint64_t k = a.key[lb + l - 1];
            const bool bad = a.fault[lb + l - 1] != 0u || k == 0ull;
            const int g = (int)~(uint32_t)k;
            const int n = a.n_nodes[r];
            int nxt = -1;
            if (!bad) {
                for (int b = prev + 1; b < n && nxt < 0; b += 64) {
                    const int u = b + lane;
                    const bool m = u < n && a.parent[rb + u] == prev && a.tokens[rb + u] == g;
                    const uint64_t bal = __ballot(m);
                    if (bal) nxt = b + __builtin_ctzll(bal);
                }
            }
            if (s == 0) {
                if (bad) {
                    for (int u = lane; u < a.M; u += 64) {
                        a.out_path[rb + u] = -1;
                        a.out_tok[rb + u] = -1;
                    }
                    if (lane == 0) atomic_or_u32(&a.ctl->status, SPEC_DEV_BAD_REQUEST);
                } else if (lane == 0) {
                    if (nxt >= 0) {
                        a.out_path[rb + l - 1] = nxt;
                        a.out_tok[rb + l - 1] = a.tokens[rb + nxt];
                        if (l < a.L) a.node[lb + l] = nxt;
                    } else {
                        a.out_tok[rb + l - 1] = g;
                        a.out_acc[r] = l - 1;
                    }
                }
            }
            if (lane == 0) cur_s = (bad || l >= a.L) ? -1 : nxt;
        }
        __syncthreads();
        cur = cur_s;
    }
    if (cur < 0) return;
    // level l: this slice of row cur
    const T *row = (const T *)a.logits + (rb + cur) * a.V;
    const int e0 = s * kTreeSlice;
    const int e1 = min(e0 + kTreeSlice, a.V);
    float v = -INFINITY;
    int idx = 0x7fffffff, bad = 0;
    if constexpr (EPV > 1) {
        // 16-byte vectors (V % EPV == 0, rows 16-byte aligned)
        constexpr int K = kTreeSlice / (kBlock * EPV);
        float z[K][EPV];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = e0 + (k * kBlock + tid) * EPV;
            VecLoad<T, EPV>::run(row, (long)(e < e1 ? e : e0), z[k]);  // in-row; masked below
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = e0 + (k * kBlock + tid) * EPV;
            if (e < e1) {
#pragma unroll
                for (int q = 0; q < EPV; ++q) tree_take(z[k][q], e + q, v, idx, bad);
            }
        }
    } else {
        for (int e = e0 + tid; e < e1; e += kBlock) tree_take(load_one(row, (long)e), e, v, idx, bad);
    }
    wave_argmax(v, idx);
    bad = wave_max_i(bad);
    if (lane == 0) {
        wv[wave] = v;
        wi[wave] = idx;
        wb[wave] = bad;
    }
    __syncthreads();
    if (tid == 0) {
        float bv = wv[0];
        int bi = wi[0], bb = wb[0];
        for (int w = 1; w < kWaves; ++w) {
            argmax_combine(bv, bi, wv[w], wi[w]);
            bb |= wb[w];
        }
        if (bb) {
            atomic_or_u32(&a.fault[lb + l], 1u);
        } else {
            // -0.0 and +0.0 are one value to the greedy rule (the lowest id
            // among equal maxima wins), so both take +0.0's word
            const uint64_t word =
                ((uint64_t)tree_ord(bv == 0.0f ? 0.0f : bv) << 32) | (uint32_t)~(uint32_t)bi;
            __hip_atomic_fetch_max(&a.key[lb + l], word, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace sv

using namespace sv;

extern "C" {

size_t spec_tree_workspace_bytes(int R, int M, int V) {
    if (R < 1 || M < 1 || M > kTreeMaxNodes || V < 1 || V > SPEC_MAX_VERIFY_VOCAB) return 0;
    // node, key and fault words for up to M levels per request
    return sizeof(Control) + (size_t)R * M * (4 + 8 + 4) + 256;
}

int spec_tree_verify(const void *logits, int dtype, const int32_t *parent, const int32_t *tokens,
                     const int32_t *n_nodes, int R, int M, int V, int max_depth,
                     int32_t *out_accepted, int32_t *out_path, int32_t *out_tokens,
                     void *workspace, size_t workspace_bytes, void *stream) {
    if (R < 0 || M < 1 || V < 1 || max_depth < 0) return SPEC_EINVAL;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
    if (M > kTreeMaxNodes || V > SPEC_MAX_VERIFY_VOCAB || max_depth >= M) return SPEC_EUNSUPPORTED;
    if (R == 0) return SPEC_OK;
    if (!logits || !parent || !tokens || !n_nodes || !out_accepted || !out_path || !out_tokens)
        return SPEC_EINVAL;
    const int L = max_depth + 1;
    const size_t need = sizeof(Control) + (size_t)R * L * (4 + 8 + 4) + 256;
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < need)
        return SPEC_EWORKSPACE;
    char *ws = (char *)workspace;
    TreeArgs a{};
    a.logits = logits;
    a.parent = parent;
    a.tokens = tokens;
    a.n_nodes = n_nodes;
    a.R = R;
    a.M = M;
    a.V = V;
    a.S = (V + kTreeSlice - 1) / kTreeSlice;
    a.max_depth = max_depth;
    a.L = L;
    a.out_acc = out_accepted;
    a.out_path = out_path;
    a.out_tok = out_tokens;
    a.key = (uint64_t *)(ws + sizeof(Control));
    a.node = (int32_t *)(ws + sizeof(Control) + 8 * (size_t)R * L);
    a.fault = (uint32_t *)(ws + sizeof(Control) + 12 * (size_t)R * L);
    a.ctl = (Control *)ws;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(tree_init_kernel, dim3((unsigned)R), dim3(64), 0, st, a);
    const size_t eb = dtype == SPEC_BF16 ? 2 : 4;
    const bool vec = (V % (16 / eb) == 0) && ((uintptr_t)logits % 16 == 0);
    const dim3 grid((unsigned)a.S, (unsigned)R);
    // levels 0 .. max_depth read a row each; launch max_depth + 1 only steps
    for (int l = 0; l <= L; ++l) {
        a.level = l;
        if (dtype == SPEC_BF16) {
            if (vec) hipLaunchKernelGGL((tree_level_kernel<uint16_t, 8>), grid, dim3(kBlock), 0, st, a);
            else hipLaunchKernelGGL((tree_level_kernel<uint16_t, 1>), grid, dim3(kBlock), 0, st, a);
        } else {
            if (vec) hipLaunchKernelGGL((tree_level_kernel<float, 4>), grid, dim3(kBlock), 0, st, a);
            else hipLaunchKernelGGL((tree_level_kernel<float, 1>), grid, dim3(kBlock), 0, st, a);
        }
    }
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
