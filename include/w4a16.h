/*
 * w4a16.h -- C ABI of the MI355X (gfx950) INT4 group-quantized weight-only
 * linear layer: 4-bit weights on a per-group scale/zero-point grid, bf16
 * activations, fp32 accumulation.
 *
 * The method (arXiv 2607.04244, "Quantize the Target, Quantize the Drafter:
 * Efficient Inference with Qwen3.5-4B"): the target model is served from an
 * AWQ INT4 checkpoint whose per-group scales stay frozen, so its weights are
 * re-packed onto the same grid and packing and serving are unchanged (Pith
 * review, Referee Report: Summary and Significance; Assumptions & free
 * parameters: frozen AWQ per-group scales).  The drafter is group-wise INT4
 * with group size 128 (Pith review, free parameters: GPTQ group size 128).
 * Each speculative step checks a block of 16 draft tokens against the target's
 * own greedy choices, which leaves the target's output unchanged (Pith review,
 * free parameters: block size 16; Assumptions & free parameters, first
 * assumption; mlsanity index page, Abstract).
 *
 * Definitions (the pages print no formula; these are the plainest readings):
 *   G = K / group                        (group must be 128)
 *   q[n,k] = (qweight[n*(K/8) + k/8] >> (4*(k%8))) & 15
 *   z[n,g] = (qzeros[(n/8)*G + g]   >> (4*(n%8))) & 15
 *   s[n,g] = scales[n*G + g]                         (IEEE binary16)
 *   W[n,k] = (q[n,k] - z[n, k/group]) * s[n, k/group]
 *   Y[m,n] = sum_k X[m,k] * W[n,k]                   (X bfloat16, fp32 accumulation)
 *
 * Conventions shared by every call:
 *   - Every pointer is device memory owned by the caller (HIP device
 *     allocations, e.g. torch tensors).  The library never allocates, frees or
 *     synchronizes; it only enqueues kernels on `stream` (a hipStream_t; NULL
 *     means the default stream).  Inputs are read-only; outputs must not
 *     alias inputs or each other.
 *   - bf16 and fp16 values cross the ABI as raw 16-bit patterns.
 *   - All arguments are checked on the host before anything is enqueued; on
 *     an error nothing is enqueued, nothing is printed, and the status code is
 *     returned.  A failed kernel launch returns W4A16_ERR_HIP.
 *   - Pointers must be 16-byte aligned (they are read with 128-bit loads).
 *   - Empty problems (M == 0 or N == 0) return W4A16_OK and enqueue nothing.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Workspace: the first 64 KiB hold arrival counters and argmax keys that
 *     must be zero when a call starts.  Zero-fill a workspace once when it is
 *     allocated; every call returns that region to zero before it completes,
 *     so one workspace serves calls of any shape in sequence.  Calls that
 *     share a workspace must be ordered (same stream, or synchronized).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum w4a16_status {
    W4A16_OK = 0,
    W4A16_ERR_NULL = 1,        /* a required pointer is NULL */
    W4A16_ERR_SHAPE = 2,       /* M, N or K out of the supported range */
    W4A16_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    W4A16_ERR_UNSUPPORTED = 4, /* group != 128, or an unknown output dtype */
    W4A16_ERR_WORKSPACE = 5,   /* workspace smaller than w4a16_workspace_bytes() */
    W4A16_ERR_HIP = 6          /* a kernel launch failed */
};

enum w4a16_out_dtype {
    W4A16_OUT_BF16 = 0, /* Y stored as bfloat16, rounded to nearest even */
    W4A16_OUT_F32 = 1   /* Y stored as the fp32 accumulator (exactness / debug mode) */
};

enum w4a16_op {
    W4A16_OP_LINEAR = 0,          /* w4a16_linear */
    W4A16_OP_LMHEAD = 1,          /* w4a16_lmhead_verify */
    W4A16_OP_LINEAR_ACTORDER = 2, /* w4a16_linear_actorder */
    W4A16_OP_LINEAR_GATED = 3     /* w4a16_linear_gated */
};

/*
 * w4a16_pack -- put 4-bit codes and zero-points onto the packed grid.
 * The pages: weights are re-packed onto the frozen AWQ grid, and packing stays
 * as it was (Pith review, Referee Report: Summary, Significance).
 *   codes  [N][K]   uint8, one code per byte; only the low 4 bits are used
 *   zeros  [N][G]   uint8, one zero-point per byte; only the low 4 bits are used
 *   qweight[N][K/8] uint32 out: nibble j (bits 4j..4j+3) of word w of row n = code (n, 8w+j)
 *   qzeros [N/8][G] uint32 out: nibble j of word (r, g) = zero of row 8r+j, group g
 * Shapes: N % 8 == 0, K % group == 0, K >= group, group == 128.
 */
int w4a16_pack(const uint8_t *codes, const uint8_t *zeros, int N, int K, int group,
               uint32_t *qweight, uint32_t *qzeros, void *stream);

/*
 * GPTQ act-order ("desc_act") support.  With act-order, column k of the weight
 * belongs to group g_idx[k] instead of k / group (the pages' drafter is GPTQ INT4
 * with groups of 128: Pith review, Assumptions & free parameters; the pages do not
 * say whether it uses act-order).  Reading: W[n,k] = (q[n,k] - z[n,g_idx[k]]) *
 * s[n,g_idx[k]]; symmetric GPTQ is z = 8 everywhere.  A permutation of the K axis
 * makes every group's columns consecutive, after which the grid is the plain one:
 *   perm[j] = the j-th column in (group, column) order, g_idx[perm[j]] = j / group.
 *
 * w4a16_actorder_perm -- the permutation, on the host (host pointers g_idx[K],
 * perm[K]).  W4A16_ERR_SHAPE unless K % group == 0, every g_idx is in
 * [0, K/group) and every group holds exactly `group` columns; W4A16_ERR_NULL.
 */
int w4a16_actorder_perm(const int32_t *g_idx, int K, int group, int32_t *perm);

/*
 * w4a16_pack_actorder -- w4a16_pack of the columns in perm order:
 * qweight[n][j/8] nibble j%8 holds codes[n][perm[j]]; qzeros as w4a16_pack.
 * codes u8[N][K] and zeros u8[N][K/group] in natural column order; perm i32[K]
 * from w4a16_actorder_perm (device copy).  Shapes and errors as w4a16_pack; perm
 * must be 16-byte aligned (an index outside [0, K) is clamped, never followed).
 */
int w4a16_pack_actorder(const uint8_t *codes, const uint8_t *zeros, const int32_t *perm, int N, int K,
                        int group, uint32_t *qweight, uint32_t *qzeros, void *stream);

/*
 * w4a16_linear_actorder -- Y = X * W^T for an act-order grid packed by
 * w4a16_pack_actorder: X [M][K] bf16 in natural column order enters the
 * contraction as X'[m][k] = X[m][perm[k]].  At M = 1 up to 40 groups the gather
 * runs inside the kernel's X staging; otherwise X' is written to the workspace first
 * and the call proceeds as w4a16_linear (same kernels, same accuracy bound).  An entry of perm outside
 * [0, K) reads X[m][K - 1].  workspace: at least
 * w4a16_workspace_bytes(W4A16_OP_LINEAR_ACTORDER, M, N, K, group) (the size of the
 * separate gather, whichever path runs).  Shapes and errors as w4a16_linear; perm
 * (device) must be 16-byte aligned.
 */
int w4a16_linear_actorder(const void *X, const int32_t *perm, const uint32_t *qweight, const void *scales,
                          const uint32_t *qzeros, int M, int N, int K, int group, void *Y, int y_dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a16_swa_attention -- causal sliding-window attention of a block of M query tokens
 * at the end of a context of T tokens: the drafter's long-context lever (Pith review,
 * Assumptions & free parameters: an SWA window of 1024 tokens on the leaderboard, 1024
 * or 2048 in the window study; the pages' Figure 1: inputs of up to 8192 tokens).  The
 * pages give no formula; reading:
 *   query i (0 <= i < M) sits at position p_i = T - M + i; head h reads key/value
 *   head h / (Hq / Hkv); it attends to keys p_i - window < j <= p_i (j >= 0):
 *   O[i,h,:] = sum_j softmax_j(Q[i,h,:] . K[j,kv,:] / sqrt(D)) V[j,kv,:]
 * fp32 scores and sums; the softmax weights enter the value product as a pair of
 * bf16 values (hi + lo, relative error about 2^-17).
 *   Q   [M][Hq][D]         bf16 (device)
 *   K   [T][Hkv][D]        bf16 key cache, token-major (device)
 *   Vt  [Hkv][D][t_stride] bf16 value cache, transposed: row (kv, d) holds the values
 *                          of dimension d for tokens 0 .. T-1 (device); t_stride >= T,
 *                          a multiple of 8; entries past T are never used
 *   O   [M][Hq][D]         bf16 or fp32 (o_dtype as y_dtype of w4a16_linear)
 *   workspace              at least w4a16_swa_workspace_bytes(M, T, Hq, Hkv, window)
 * Shapes: D == 128 (else W4A16_ERR_UNSUPPORTED), 1 <= M <= 16, M <= T, Hq a multiple
 * of Hkv with Hq / Hkv <= 16, 1 <= window <= 65536; element counts at most 2^31 - 256.
 * Errors: W4A16_ERR_SHAPE, _UNSUPPORTED, _NULL, _ALIGN (16 bytes), _WORKSPACE, _HIP.
 */
int w4a16_swa_attention(const void *Q, const void *K, const void *Vt, int M, int T, int Hq, int Hkv, int D,
                        int window, int t_stride, void *O, int o_dtype, void *workspace, size_t workspace_bytes,
                        void *stream);
size_t w4a16_swa_workspace_bytes(int M, int T, int Hq, int Hkv, int window);

/*
 * w4a16_swa_attention_block -- as w4a16_swa_attention, bidirectional within the block:
 * the drafter proposes a whole block of tokens at once (mlsanity index page, Builds
 * on: block diffusion for speculative decoding; Pith review, What carries the
 * argument), so each query attends to every key of the block and to the context
 * keys inside its window.  Reading: query i (position p_i = T - M + i) sees keys
 * T - M <= j < T and p_i - window < j < T - M (j >= 0).  Arguments, layouts,
 * workspace (w4a16_swa_workspace_bytes), shapes and errors as w4a16_swa_attention.
 */
int w4a16_swa_attention_block(const void *Q, const void *K, const void *Vt, int M, int T, int Hq, int Hkv, int D,
                              int window, int t_stride, void *O, int o_dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * w4a16_quantize -- round a weight matrix back onto the grid, keeping the grid's
 * per-group scales and zero-points: the re-packing step of the pages'
 * distillation, which keeps the INT4 grid's scales fixed so that the packed format
 * and the serving path do not change (Pith review, Referee Report: Summary and
 * Significance; Assumptions & free parameters, second assumption).  The pages give
 * no formula; this is the asymmetric reading, the inverse of W = (q - z) * s:
 *     q[n,k] = clamp(round(W[n,k] / s[n,g]) + z[n,g], 0, 15),  g = k / group
 * round = the exact quotient to the nearest integer, ties to even, applied before z
 * is added.  The codes are written packed (no unpacked copy is made).
 *   W        [N][K]    bf16 weights, row-major (device)
 *   scales   [N][G]    fp16 (device, frozen)
 *   qzeros   [N/8][G]  uint32, layout of w4a16_pack (device, frozen)
 *   qweight  [N][K/8]  uint32 out, layout of w4a16_pack (device; must not alias)
 * Shapes: N >= 0, N % 8 == 0, K >= group, K % group == 0, group == 128,
 *         N * K at most 2^31 - 256.  N == 0 enqueues nothing.
 * Errors: W4A16_ERR_SHAPE, W4A16_ERR_UNSUPPORTED (group), W4A16_ERR_NULL,
 *         W4A16_ERR_ALIGN (16-byte alignment), W4A16_ERR_HIP.
 */
int w4a16_quantize(const void *W, const void *scales, const uint32_t *qzeros, int N, int K, int group,
                   uint32_t *qweight, void *stream);

/*
 * w4a16_linear -- Y[M][N] = X[M][K] * W^T on the grid defined above.
 * The layer the pages' INT4 target and GPTQ-INT4 drafter spend their forward
 * passes in (Pith review, Referee Report: Summary; free parameters: group 128).
 *   X        [M][K]    bf16, row-major
 *   qweight  [N][K/8]  uint32 (layout of w4a16_pack)
 *   scales   [N][G]    fp16
 *   qzeros   [N/8][G]  uint32
 *   Y        [M][N]    row-major, bf16 (W4A16_OUT_BF16) or fp32 (W4A16_OUT_F32)
 *   workspace          device scratch of at least
 *                      w4a16_workspace_bytes(W4A16_OP_LINEAR, M, N, K, group) bytes;
 *                      its counter region must hold zeros before its first
 *                      use (allocate it zero-filled); every call returns that
 *                      region to zero.
 *                      May be NULL when that size is 0.
 * Shapes: M >= 0, N >= 0, N % 8 == 0, K >= group, K % group == 0, group == 128,
 *         M * N, N * K and M * K at most 2^31 - 256.
 */
int w4a16_linear(const void *X, const uint32_t *qweight, const void *scales, const uint32_t *qzeros,
                 int M, int N, int K, int group, void *Y, int y_dtype,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a16_linear_static_ws -- w4a16_linear for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same kernels and result bits as w4a16_linear with a fresh
 * zero-filled workspace; the scratch memory is instead a per-device array inside
 * the library of W4A16_STATIC_WS_BYTES, held by every GPU the library runs on
 * until the process ends.  The caller passes inputs and outputs only.
 *   X, qweight, scales, qzeros, Y, y_dtype, stream   as w4a16_linear
 * The array belongs to the device current on the calling thread.  Its first call
 * there obtains the array's address and clears its counter region with a kernel
 * enqueued on `stream`; every call returns that region to zero.  All calls on one
 * GPU share the array, which keeps the last call's contents: calls that overlap on
 * one GPU (unordered streams, or threads) race and must be serialized by the caller.
 * Nothing is allocated or freed, here or in any call below it.
 * Errors: those of w4a16_linear; W4A16_ERR_WORKSPACE when the shape needs more
 * scratch than the array holds, i.e. when
 * w4a16_workspace_bytes(W4A16_OP_LINEAR, M, N, K, group) > W4A16_STATIC_WS_BYTES
 * (the M > 64 path needs 2 M K bytes and more); W4A16_ERR_HIP when the array's
 * address cannot be obtained or a launch fails.
 */
#define W4A16_STATIC_WS_BYTES (8u << 20)
int w4a16_linear_static_ws(const void *X, const uint32_t *qweight, const void *scales, const uint32_t *qzeros,
                           int M, int N, int K, int group, void *Y, int y_dtype, void *stream);

/*
 * w4a16_linear_gated -- the gate and up projections of a gated MLP and its
 * activation in one call: Y = silu(X * Wg^T) * (X * Wu^T), elementwise, with
 * silu(g) = g / (1 + exp(-g)).  The pages serve a Qwen3.5-4B target (Pith review,
 * Referee Report: Summary) and do not spell out its MLP; the gated form, with the
 * activation applied to the fp32 sums of both projections, is that family's MLP
 * (a reading).  Wg and Wu are two grids of the layouts of w4a16_linear over the
 * same N columns.  For M <= 64 one launch computes both projections (each
 * workgroup holds a gate tile and the up tile of the same columns) and applies the
 * activation in its epilogue, so neither projection's output reaches memory; so
 * does the large-M tile kernel when its tiles of 256 rows x 128 columns fill the
 * GPU's compute units at least once.  In between, the two projections run in turn
 * into the workspace (fp32) and a third kernel applies the activation.
 *   X                                     [M][K] bf16, row-major
 *   qweight_gate, scales_gate, qzeros_gate   the gate grid (layouts of w4a16_linear)
 *   qweight_up, scales_up, qzeros_up         the up grid, same N and K
 *   Y                                     [M][N] row-major, bf16 or fp32
 *   workspace   at least w4a16_workspace_bytes(W4A16_OP_LINEAR_GATED, M, N, K, group)
 *               bytes (M > 64: X as scaled fp16, and in the in-between range the
 *               fp32 outputs of both projections); the
 *               counter-region rule of w4a16_linear; may be NULL when that size is 0
 * Shapes: as w4a16_linear, and N % 16 == 0, 2 * M * N at most 2^31 - 256.
 * Errors: as w4a16_linear (W4A16_ERR_SHAPE also for N % 16 != 0).  Y must not
 * alias any input.
 */
int w4a16_linear_gated(const void *X, const uint32_t *qweight_gate, const void *scales_gate,
                       const uint32_t *qzeros_gate, const uint32_t *qweight_up, const void *scales_up,
                       const uint32_t *qzeros_up, int M, int N, int K, int group, void *Y, int y_dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a16_linear_batch -- several projections of the same rows in one launch.
 * Verifying a draft block of 16 tokens runs every projection of a decoder layer on
 * 16 rows (Pith review, free parameters: block size 16), and a decode step runs
 * them on one row; each projection alone is too small to fill the GPU or to hide a
 * launch.  This call computes Y_q = X_q * W_q^T for every entry of
 * problems[0 .. count) as w4a16_linear would (same grid, same reading, same
 * accuracy bound), in one launch when M <= 64 (one after another when M > 64).
 * At M = 1, entries that share X and K run as one launch of the decode kernel, each
 * with its own run of workgroups, and give the same bits as single calls.
 *   problems  host array of count descriptors (read during the call only); each
 *             names its own device tensors X [M][K] bf16, qweight, scales, qzeros,
 *             Y [M][N], and its N and K (the layouts of w4a16_linear)
 *   count     0 .. W4A16_MAX_BATCH
 *   M, group, y_dtype   shared by all entries
 *   workspace at least the sum over the entries of
 *             w4a16_workspace_bytes(W4A16_OP_LINEAR, M, N_q, K_q, group) (projections
 *             that split K across workgroups keep their partial sums side by side);
 *             the rules of w4a16_linear
 * Errors: as w4a16_linear, checked for every entry before anything is launched;
 * W4A16_ERR_SHAPE also for count outside 0 .. W4A16_MAX_BATCH.  Entries with N == 0
 * and calls with M == 0 do nothing.  Outputs must not alias each other or inputs.
 */
#define W4A16_MAX_BATCH 8
typedef struct w4a16_problem {
    const void *X;            /* bf16 [M][K] */
    const uint32_t *qweight;  /* [N][K/8] */
    const void *scales;       /* fp16 [N][K/group] */
    const uint32_t *qzeros;   /* [N/8][K/group] */
    void *Y;                  /* [M][N], bf16 or fp32 */
    int N, K;
} w4a16_problem;

int w4a16_linear_batch(const w4a16_problem *problems, int count, int M, int group, int y_dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a16_lmhead_verify -- the lm_head projection fused with greedy verification
 * of a draft block (Pith review, Assumptions & free parameters: the first
 * assumption, on verification; free parameters: block size 16).
 * Computes the logits Y = X * W^T as w4a16_linear does (kept in fp32), then
 *   argmax[m]   = the smallest n attaining max_n Y[m,n]   (over the fp32 logits)
 *   accept_len  = the number of leading rows i with argmax[i] == draft_ids[i]
 * Row i of X is the hidden state whose next token is compared with draft_ids[i]
 * (the caller aligns the positions).  When accept_len < M, argmax[accept_len]
 * is the target's correction token.
 *   draft_ids  [M] int32 device; values are only compared, never used as indices
 *   Y_or_null  [M][N] optional logits out (bf16 or fp32 per y_dtype), or NULL
 *   argmax     [M] int32 out;  accept_len [1] int32 out
 *   workspace  at least w4a16_workspace_bytes(W4A16_OP_LMHEAD, M, N, K, group)
 *              bytes, zero-filled before first use; every call leaves it zeroed.
 * Shapes: as w4a16_linear, plus 1 <= M <= 64 and N >= 1.
 */
int w4a16_lmhead_verify(const void *X, const uint32_t *qweight, const void *scales,
                        const uint32_t *qzeros, int M, int N, int K, int group,
                        const int32_t *draft_ids, void *Y_or_null, int y_dtype,
                        int32_t *argmax, int32_t *accept_len,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a16_workspace_bytes -- scratch size a call of `op` needs for this shape
 * (split-K partial sums, arrival counters, per-row argmax keys).  Returns 0 for
 * shapes the call would reject or that need no scratch.
 */
size_t w4a16_workspace_bytes(int op, int M, int N, int K, int group);

/* Human-readable name of a status code (static storage; never NULL). */
const char *w4a16_status_string(int status);

/* ABI version: major * 100 + minor. */
int w4a16_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
