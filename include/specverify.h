/*
 * specverify.h -- C ABI of the MI355X (gfx950) library for batched lossless
 * speculative-sampling verification and the first-order Markov-head draft.
 *
 * The method (sources cited by page title and section):
 *  - DART reading note (zhongzhuzhou.org, "DART：把草稿并行生成之后，还要补上
 *    哪些依赖？"), sec. 2.3, eq. (3)-(4): accept a draft token x with
 *    probability min(1, q(x)/p(x)); on rejection draw from the residual
 *    [q - p]_+ / R, R = sum_v [q - p]_+ = 1 - sum_v min(p, q); no residual is
 *    needed when R = 0; at temperature 0 verification compares with the
 *    target argmax.
 *  - DSpark paper guide (personal-site-bgy.pages.dev), "speculative decoding
 *    basics": gamma drafts verified in one target pass, strict left-to-right
 *    prefix survival, one bonus token from the target when every draft passes;
 *    "confidence head": the analytic acceptance rate c* = 1 - 1/2 ||p - q||_1;
 *    "scheduler": a verify length l_r per request, verify batch sum(1 + l_r);
 *    "Markov head": p_k(v | x_0, x_<k) = softmax(U_k(v) + W1[x_{k-1}] W2(v)),
 *    W1 in R^{V x r}, W2 in R^{r x V}, r = 256, x_0 the anchor token.
 *  - Speculative-decoding survey (zhifeiding.github.io), sec. 1.2-1.3 and
 *    2.1: one corrected token at the first rejection, tau = N + 1 tokens per
 *    cycle, greedy verification as a position-wise argmax comparison.
 *
 * Notation: q = target distribution, p = draft distribution, both softmaxes
 * of logits divided by the request's temperature T (T = 0: greedy).
 *
 * Conventions for every entry point:
 *  - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronises (except spec_get_device_status;
 *    spec_verify_batch_noalloc uses a fixed array of its own, see there),
 *    and enqueues its work on `stream` (a hipStream_t passed as void*; NULL is
 *    the null stream).  Calls return once the work is enqueued.
 *  - Arrays are dense and row-major with the last dimension contiguous; logit
 *    rows are fp32 or bf16 (spec_dtype).
 *  - Host-checkable faults (null required pointer, negative size, unknown
 *    dtype, workspace too small or not 256-byte aligned, unsupported shape)
 *    return a negative spec_status before anything is enqueued.  A failed
 *    kernel launch returns SPEC_EHIP.
 *  - Data faults are found on the device, per request: l_r outside [0, gamma],
 *    T negative / NaN / infinite / outside [1e-30, 1e30] when nonzero, a draft
 *    token outside [0, V), a uniform outside [0, 1), a NaN or +inf logit, or a
 *    logit row that is entirely -inf.  Such a request gets num_accepted = -1,
 *    tokens -1 and NaN floats, and SPEC_DEV_BAD_REQUEST is set in the
 *    workspace's status word.  Other requests are unaffected.  -inf logits
 *    (masked ids) are valid.
 *  - A workspace is a device buffer of at least the queried size, 256-byte
 *    aligned, initialised once with spec_workspace_init before its first use.
 *    The library keeps it consistent afterwards.  Calls that share a
 *    workspace must be ordered (same stream, or synchronised); calls with
 *    distinct workspaces may run concurrently.
 *  - Graph capture: every compute entry point may be captured into a HIP
 *    graph and replayed (device state is cleared with kernels, not memset
 *    nodes, and the verification calls draw their launch tag on the device).
 *    A workspace's status word is cleared only by spec_get_device_status.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

typedef enum {
    SPEC_OK = 0,
    SPEC_EINVAL = -1,        /* null required pointer or negative size            */
    SPEC_EDTYPE = -2,        /* dtype not supported for this argument            */
    SPEC_EWORKSPACE = -3,    /* workspace null, too small or misaligned          */
    SPEC_EHIP = -4,          /* a HIP runtime call or kernel launch failed       */
    SPEC_EUNSUPPORTED = -5,  /* shape outside the supported range                */
    SPEC_ETOOLARGE = -6      /* the call needs more than the fixed scratch of
                                spec_verify_batch_noalloc                        */
} spec_status;

/* Bits of the device status word kept in the workspace. */
#define SPEC_DEV_BAD_REQUEST 0x1u   /* a request had invalid data (see above)      */
#define SPEC_DEV_SPIN_TIMEOUT 0x2u  /* a word written by an earlier launch of the
                                       call was still stale after a bounded re-poll
                                       (an earlier launch failed); the outputs of
                                       that call are undefined                     */

/* Largest vocabulary the Markov-draft kernels accept. */
#define SPEC_MAX_VOCAB 2097152
/* Largest vocabulary spec_verify_batch and spec_tv_accept_rate accept (a row
 * is cut into at most 256 chunks of 1024 logits). */
#define SPEC_MAX_VERIFY_VOCAB 262144

/* Largest backbone hidden size spec_rnn_draft_sample accepts. */
#define SPEC_RNN_MAX_HIDDEN 3072

/* Largest candidate pool (R * gamma, and R) spec_schedule_verify_len accepts. */
#define SPEC_SCHED_MAX_POOL 8192

/* Limits of spec_sts_calibrate: bins, grid points, held-out blocks. */
#define SPEC_STS_MAX_BINS 24
#define SPEC_STS_MAX_GRID 1024
#define SPEC_STS_MAX_BLOCKS (1 << 24)

/* Largest tree (nodes per request) spec_tree_verify accepts. */
#define SPEC_TREE_MAX_NODES 1024

/* Library version, major * 10000 + minor * 100 + patch. */
int spec_version(void);

/* Human-readable name of a spec_status value (static string). */
const char *spec_status_string(int status);

/* Workspace bytes for spec_verify_batch at these sizes (0 if the sizes are
 * negative or unsupported).  The same buffer may serve every entry point as
 * long as it is large enough for each call. */
size_t spec_verify_workspace_bytes(int R, int gamma, int V);

/* Zero-fills a workspace (one small kernel on `stream`).  Call once on a new
 * buffer, or to recover a buffer after SPEC_DEV_SPIN_TIMEOUT. */
int spec_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Which launch sequence a spec_verify_batch call of this shape takes on the
 * current device, for 16-byte aligned logit rows (a negative spec_status for
 * invalid or unsupported shapes):
 *   SPEC_PATH_SPLIT  four launches: chunk statistics, normaliser folds, the
 *                    total-variation pass (which reads every row pair a second
 *                    time), the per-request combine;
 *   SPEC_PATH_HELD   two launches: one workgroup per row pair keeps most of
 *                    the pair on the compute unit between the statistics and
 *                    the total-variation pass (bf16 rows of more than 64
 *                    chunks of 1024 logits, at most 2 x compute units
 *                    candidate pairs), then the combine.
 * Both produce the same bits.  SPECVERIFY_SPLIT=1 in the environment selects
 * the split path for every call (for comparisons).  Host only; enqueues
 * nothing. */
#define SPEC_PATH_SPLIT 0
#define SPEC_PATH_HELD 1
int spec_verify_path(int R, int gamma, int V, int target_dtype, int draft_dtype);

/*
 * Batched verification (DART note eq. (3)-(4); DSpark guide "basics",
 * "confidence head", "scheduler"; survey sec. 1.3).
 *
 * For request r with l = verify_len[r], T = temperature[r], x_{i+1} =
 * draft_tokens[r][i]:
 *   T > 0:  for i < l: accept_i <=> q_i(x) >= p_i(x) or u_accept[r][i] <
 *           q_i(x)/p_i(x).  A_r = number of leading accepts.  If A_r < l the
 *           next token is an inverse-CDF draw (ascending token id, first id
 *           whose running sum exceeds u * total) from [q_A - p_A]_+ with
 *           u_sample[r][A_r] (from q_A if that residual mass is exactly 0);
 *           otherwise from q_l (target row l) with u_sample[r][l].
 *   T = 0:  g_i = argmax of target row i (lowest id on ties); accept_i <=>
 *           x == g_i; the next token is g_{A_r}.  Uniforms are not read.
 * Rows read: target rows 0..l, draft rows 0..l-1; other rows are never read.
 *
 *   target_logits  [R][gamma+1][V]  t_dtype   row i <-> draft position i+1,
 *                                             row gamma the bonus row
 *   draft_logits   [R][gamma][V]    d_dtype   (may be NULL when gamma == 0)
 *   draft_tokens   [R][gamma]   int32         (may be NULL when gamma == 0)
 *   verify_len     [R]          int32         0 <= l_r <= gamma
 *   temperature    [R]          fp32          T >= 0
 *   u_accept       [R][gamma]   fp32 in [0,1) (may be NULL when gamma == 0)
 *   u_sample       [R][gamma+1] fp32 in [0,1)
 *   out_tokens       [R][gamma+1] int32: x_1..x_A, then the drawn token, then -1
 *   out_num_accepted [R]          int32: A_r (tokens committed = A_r + 1)
 *   out_cstar        [R][gamma]   fp32, nullable: c*_i = sum_v min(p_i, q_i) for
 *                                 i < l_r (T = 0: [argmax draft == g_i]), NaN beyond
 *   out_resid_mass   [R][gamma]   fp32, nullable: sum_v [q_i - p_i]_+ (T = 0:
 *                                 1 - c*_i), NaN beyond l_r
 *   out_logq         [R][gamma+1] fp32, nullable: natural log of q_j at the
 *                                 committed token j <= A_r (0 at T = 0), NaN beyond
 * Sizes: R >= 0, 0 <= gamma <= 64, 1 <= V <= SPEC_MAX_VERIFY_VOCAB.  R == 0
 * enqueues nothing.
 */
int spec_verify_batch(const void *target_logits, int t_dtype,
                      const void *draft_logits, int d_dtype,
                      const int32_t *draft_tokens, const int32_t *verify_len,
                      const float *temperature, const float *u_accept, const float *u_sample,
                      int R, int gamma, int V,
                      int32_t *out_tokens, int32_t *out_num_accepted,
                      float *out_cstar, float *out_resid_mass, float *out_logq,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * spec_verify_batch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, outputs, dtypes, the order
 * of work on `stream` and every result are those of spec_verify_batch; the
 * workspace is instead a fixed device array inside the library, one per
 * device, SPEC_NOALLOC_SCRATCH_BYTES long, taken at its device address on the
 * first call on that device and held until the process ends.  The call makes
 * no allocation (device or host).
 * Limits: a call whose workspace (spec_verify_workspace_bytes(R, gamma, V))
 * exceeds SPEC_NOALLOC_SCRATCH_BYTES returns SPEC_ETOOLARGE before enqueueing
 * anything.  Every call on one device shares that device's array: calls that
 * may overlap on one device (different streams, or different host threads
 * without ordering) race and must not be issued; calls ordered on one stream
 * are fine.  The array keeps the last call's contents; each call's words
 * carry that call's tag, so nothing needs clearing between calls.  Device-side
 * data faults still mark the faulty request's outputs (num_accepted = -1,
 * tokens -1, NaN floats); the status bits themselves stay in the library's
 * array and are not reported.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (32u << 20)
int spec_verify_batch_noalloc(const void *target_logits, int t_dtype,
                              const void *draft_logits, int d_dtype,
                              const int32_t *draft_tokens, const int32_t *verify_len,
                              const float *temperature, const float *u_accept,
                              const float *u_sample, int R, int gamma, int V,
                              int32_t *out_tokens, int32_t *out_num_accepted,
                              float *out_cstar, float *out_resid_mass, float *out_logq,
                              void *stream);

/*
 * Measurement hook.  For the next n verification calls (spec_verify_batch,
 * spec_verify_batch_noalloc, spec_tv_accept_rate) made by the calling host
 * thread, the library records the events before[i] and after[i] (hipEvent_t
 * passed as void*, created and owned by the caller) on the call's stream
 * immediately before and after its first launch -- the one that streams
 * every needed logit row from HBM: the statistics launch on the split path,
 * the held-pair launch on the held path (spec_verify_path) -- so that the
 * caller can time that kernel alone (hipEventElapsedTime).  The arrays must
 * stay valid until
 * those n calls have been made; n = 0 stops.  Returns SPEC_EINVAL for n < 0
 * or missing arrays.
 */
int spec_time_stats_launch(void *const *before, void *const *after, int n);

/* Workspace bytes for spec_tv_accept_rate. */
size_t spec_tv_workspace_bytes(int N, int V);

/*
 * Analytic acceptance rate of N independent row pairs (DSpark guide,
 * "confidence head": c* = 1 - 1/2 ||p - q||_1; DART note eq. (3)).
 *   draft_logits, target_logits  [N][V]  dtype
 *   temperature                  [N]     fp32 (T = 0: c* = [argmax p == argmax q])
 *   out_cstar                    [N]     fp32 = sum_v min(p, q)
 *   out_resid_mass               [N]     fp32, nullable = sum_v [q - p]_+
 * Invalid rows (data faults as above) give NaN and set SPEC_DEV_BAD_REQUEST.
 */
int spec_tv_accept_rate(const void *draft_logits, const void *target_logits, int dtype,
                        const float *temperature, int N, int V,
                        float *out_cstar, float *out_resid_mass,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for spec_markov_draft_sample. */
size_t spec_markov_workspace_bytes(int R, int gamma, int V, int rank);

/*
 * First-order Markov-head draft (DSpark guide, "Markov head"), serial over
 * k = 1..gamma for every request r, with x_0 = anchor[r]:
 *   l_k(v) = fp32( U[r][k-1][v] + sum_j W1[x_{k-1}][j] W2[j][v] )
 *   x_k    = inverse-CDF draw (ascending id) from softmax(l_k / T_r) with
 *            u_draft[r][k-1]; argmax of l_k (lowest id) at T_r = 0.
 * The stored fp32 logits are the draft distribution that verification must
 * compare against (pass out_draft_logits as draft_logits, d_dtype SPEC_F32).
 *   U              [R][gamma][V]  u_dtype (fp32 or bf16)
 *   W1             [V][rank]      w_dtype (bf16), 16-byte aligned
 *   W2             [rank][V]      w_dtype (bf16), 16-byte aligned
 *   anchor         [R]            int32 in [0, V)
 *   temperature    [R]            fp32
 *   u_draft        [R][gamma]     fp32 in [0,1)
 *   out_draft_tokens [R][gamma]   int32 (-1 for an invalid request)
 *   out_draft_logits [R][gamma][V] fp32
 * Sizes: R >= 0, gamma >= 0, 1 <= V <= SPEC_MAX_VOCAB, rank == 256.
 * A misaligned W1 or W2 returns SPEC_EINVAL.
 * Per step: one logits launch over 64-id tiles (a persistent launch over
 * 128-id tiles where R == 64 and the rows allow 16-byte accesses), then one
 * draw launch.  Both logits launches produce the same bits;
 * SPECMARKOV_TILES=1 in the environment selects the per-tile one for every
 * call (for comparisons).
 */
int spec_markov_draft_sample(const void *U, int u_dtype,
                             const void *W1, const void *W2, int w_dtype,
                             const int32_t *anchor, const float *temperature,
                             const float *u_draft,
                             int R, int gamma, int V, int rank,
                             int32_t *out_draft_tokens, float *out_draft_logits,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for spec_rnn_draft_sample. */
size_t spec_rnn_workspace_bytes(int R, int gamma, int V, int rank, int hidden);

/*
 * RNN serial head (DSpark guide, the serial-head section: the RNN variant
 * described after the Markov head).
 *
 * Like spec_markov_draft_sample, with the transition bias taken from a
 * recurrent state instead of the previous token alone: s_0 = 0 and, for
 * k = 1..gamma, with c = [s_{k-1}; W1[x_{k-1}]; h_k] (2 rank + hidden values),
 *   z   = sigmoid(c Wg[:, 0:rank] + bg[0:rank])
 *   n   = tanh(c Wg[:, rank:2 rank] + bg[rank:2 rank])
 *   s_k = (1 - z) * s_{k-1} + z * n                      (fp32)
 *   l_k = U_k + s_k W2,  x_k ~ softmax(l_k / T)           (as the Markov head)
 * The product s_k W2 runs on the bf16 MFMA with s_k split into three bf16
 * parts (hi + mid + lo = s_k to fp32 precision).  The pages fix no gate
 * form; this single update gate on the concatenation is the reading taken.
 *   hidden_states [R][gamma][hidden]     fp32 backbone hidden states h_k
 *   Wg            [2 rank + hidden][2 rank]  w_dtype (bf16), 16-byte aligned
 *   bg            [2 rank]               fp32
 *   out_state     [R][gamma][rank]       fp32 states s_k, nullable
 * Other arguments, sizes and errors as spec_markov_draft_sample, plus
 * 1 <= hidden <= SPEC_RNN_MAX_HIDDEN; a misaligned Wg returns SPEC_EINVAL.
 */
int spec_rnn_draft_sample(const void *U, int u_dtype, const void *W1, const void *W2,
                          int w_dtype, const float *hidden_states, int hidden, const void *Wg,
                          const float *bg, const int32_t *anchor, const float *temperature,
                          const float *u_draft, int R, int gamma, int V, int rank,
                          int32_t *out_draft_tokens, float *out_draft_logits, float *out_state,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for spec_schedule_verify_len (the device status word). */
size_t spec_schedule_workspace_bytes(void);

/*
 * Confidence-scheduled verify lengths (DSpark guide, "scheduler").
 *
 * The survival probability of draft position j of request r is the running
 * product a[r][j] = c[r][1] * ... * c[r][j] of the confidence head's outputs
 * (fp32, left to right).  All candidates (r, j) form one pool in descending
 * a (ties: request, then position ascending).  Starting from l_r = 0 for
 * every request (B = R, tau = R), candidates are admitted in pool order,
 * each adding 1 to B and a[r][j] to tau (fp64), and
 *   topk < 0:  the walk stops at the first admission after which
 *              Theta = tau * sps[B] is not larger than before it (the early
 *              stop of the pages' greedy scheduler);
 *   topk >= 0: the first topk candidates are admitted (the asynchronous
 *              top-K variant), with no comparison.
 * Either walk also stops before B would pass bmax.  out_len[r] is the number
 * of admitted positions of request r (always a prefix).
 *   confidence  [R][gamma]  fp32 in [0, 1]      (device)
 *   sps         [bmax + 1]  fp32 >= 0, finite   (device; steps per second at
 *                                                batch size B, index B)
 *   out_len     [R]         int32               (device)
 *   out_theta   [1]         fp64, nullable      (device; Theta of the result)
 * Sizes: R >= 0, gamma >= 0, bmax >= 0, R * gamma <= SPEC_SCHED_MAX_POOL.
 * A confidence outside [0, 1] (or NaN) or a negative or non-finite table
 * entry sets SPEC_DEV_BAD_REQUEST in the workspace status word and every
 * out_len to -1.  One workgroup; the inputs, outputs and workspace belong to
 * the caller; work is enqueued on `stream`.
 */
int spec_schedule_verify_len(const float *confidence, const float *sps, int R, int gamma,
                             int bmax, int topk, int32_t *out_len, double *out_theta,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for spec_sts_calibrate (0 for sizes it does not accept). */
size_t spec_sts_workspace_bytes(int N, int gamma, int G, int bins);

/*
 * Sequential temperature scaling of the confidence head (DSpark guide, the
 * confidence-head section, "STS"), on a held-out set of N draft blocks.
 *
 * Position k's score of block n is c = sigmoid(z[n][k] / t_k); the
 * cumulative probability a_k = c_1 ... c_k is labelled by
 * y_k = [accepted_len[n] >= k] (positions 1..k all accepted).  Left to right,
 * t_k is the grid temperature minimising
 *   ECE_k(t) = sum_m |sum_{n in bin m} (a_{n,k}(t) - y_{n,k})| / N
 * over `bins` equal-width bins of [0, 1] (a value of 1 in the last bin), with
 * t_1..t_{k-1} fixed; ties go to the first grid point.  All arithmetic is
 * fp64 in a fixed order.  The pages give the search, not these details: the
 * sigmoid form, the prefix label, the bin layout and the tie rule are the
 * readings taken.  A grid of the single value 1 reports the raw scores' ECE.
 *   conf_logits     [N][gamma]  fp32 raw head logits, finite  (device)
 *   accepted_len    [N]         int32 in [0, gamma]           (device)
 *   grid            [G]         fp64 temperatures > 0         (device)
 *   out_temperature [gamma]     fp64                          (device)
 *   out_ece         [gamma]     fp64, ECE at the chosen t     (device)
 *   out_curve       [gamma][G]  fp64 ECE at every grid point, nullable
 * Sizes: N >= 0, gamma >= 0, 1 <= G <= SPEC_STS_MAX_GRID,
 * 1 <= bins <= SPEC_STS_MAX_BINS, N <= SPEC_STS_MAX_BLOCKS.  A non-finite
 * logit, an accepted length outside [0, gamma] or a grid value that is not a
 * positive finite number sets SPEC_DEV_BAD_REQUEST and makes every output
 * NaN.  The inputs, outputs and workspace belong to the caller; work is
 * enqueued on `stream`.
 */
int spec_sts_calibrate(const float *conf_logits, const int32_t *accepted_len, const double *grid,
                       int N, int gamma, int G, int bins, double *out_temperature,
                       double *out_ece, double *out_curve, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Workspace bytes for spec_tree_verify (0 for sizes it does not accept). */
size_t spec_tree_workspace_bytes(int R, int M, int V);

/*
 * Greedy (T = 0) verification of draft trees (speculative-decoding survey,
 * sec. 2.3, tree drafting; DART reading note, sec. 2.3: at temperature zero
 * the target argmax is followed along the candidate paths -- the pages give
 * no rule for T > 0, and none is offered).
 *
 * Request r's tree has n_nodes[r] nodes in topological order: node 0 is the
 * root (the last committed token), node v >= 1 has parent[r][v] in [0, v)
 * and draft token tokens[r][v]; logits[r][v] is the target's next-token row
 * after the path root .. v.  From the root, the walk moves to the child whose
 * token equals the argmax of the current row (lowest id on ties; the
 * lowest-index child among equal siblings) and stops at a node with no such
 * child; that row's argmax is the bonus or correction token.  Only the rows
 * on the accepted path are read, one launch per level (max_depth + 2).
 *   logits       [R][M][V]  dtype (SPEC_F32 / SPEC_BF16)    (device)
 *   parent       [R][M]     int32 (root and slots >= n_nodes ignored)
 *   tokens       [R][M]     int32 in [0, V)
 *   n_nodes      [R]        int32 in [1, M]
 *   max_depth    a bound on every tree's depth, 0 <= max_depth < M (a deeper
 *                tree is rejected as malformed)
 *   out_accepted [R]        int32 accepted draft nodes A_r
 *   out_path     [R][M]     int32 the accepted nodes in order, -1 padded
 *   out_tokens   [R][M]     int32 the A_r path tokens, then the bonus, -1 padded
 * Sizes: R >= 0, 1 <= M <= SPEC_TREE_MAX_NODES, 1 <= V <= SPEC_MAX_VERIFY_VOCAB.
 * A malformed tree (a parent outside [0, v), a token outside [0, V), n_nodes
 * outside [1, M], depth beyond max_depth) or a row on the walk holding a NaN
 * or +-inf logit sets SPEC_DEV_BAD_REQUEST and gives that request
 * out_accepted -1 and all-(-1) paths and tokens.  The inputs, outputs and
 * workspace belong to the caller; work is enqueued on `stream`.
 */
int spec_tree_verify(const void *logits, int dtype, const int32_t *parent, const int32_t *tokens,
                     const int32_t *n_nodes, int R, int M, int V, int max_depth,
                     int32_t *out_accepted, int32_t *out_path, int32_t *out_tokens,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Synchronises `stream`, copies the workspace's device status word (the OR
 * of SPEC_DEV_* bits raised since the last clear) to *host_bits, and clears
 * it when `clear` is nonzero. */
int spec_get_device_status(void *workspace, uint32_t *host_bits, int clear, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
