/*
 * fa.h -- C ABI of libfa: exact scaled-dot-product attention on MI355X (gfx950).
 *
 * The operation (cited by page title and section):
 *   Forward:  O = softmax(scale * Q K^T + M) V, with the causal mask
 *             M_ij = -inf for j > i ("CUDA FlashAttention: from online softmax
 *             to the long-sequence IO limit", §1), computed tile by tile with
 *             the online-softmax recurrence (same page, §4; "Why FlashAttention
 *             does not need to store the attention matrix", §3.2) so that the
 *             score and probability matrices never reach device memory.  The
 *             per-row log-sum-exp LSE_i = m_i + ln(l_i) (natural log) is
 *             emitted for the backward pass ("Why FlashAttention ...", §3.2
 *             and §3.3).
 *   Backward: recomputes P = exp(scale * Q K^T + M - LSE) tile by tile and
 *             forms dV = P^T dO, dP = dO V^T, dS = P * (dP - Delta),
 *             dQ = scale * dS K, dK = scale * dS^T Q, with
 *             Delta_i = sum_d dO_id O_id ("Why FlashAttention ...", §3.3;
 *             "FlashAttention algorithm details", §4.3.1-4.3.2; the
 *             correction term of "FlashAttention dataflow and engineering
 *             validation on MI50", §3.3).
 *
 * Memory and layout (all entry points):
 *   - Every tensor pointer is a DEVICE pointer into memory the caller owns.
 *     The library never allocates, frees or synchronises; it enqueues kernels
 *     on `stream` (a hipStream_t; NULL means the default stream) and returns.
 *   - Q, K, V, O, dO, dQ, dK, dV: contiguous row-major [B, H, N, D], D fastest,
 *     element type fp16 (FA_FP16) or bf16 (FA_BF16), 16-byte aligned base.
 *   - LSE and the backward workspace: contiguous FP32 [B, H, N], 16-byte
 *     aligned.
 *   - Outputs must not alias inputs or each other.
 *   - Supported: D in {64, 128}; any 1 <= N <= 2^30; B, H >= 1;
 *     B*H*ceil(N/64) < 2^31; scale finite and >= 2^-64 (the backward
 *     keeps -LSE/scale in FP32).  Anything else is
 *     rejected with an error code before any work is enqueued -- never
 *     silently computed ("CUDA FlashAttention ...", §9: unsupported shapes
 *     fall back explicitly).
 *   - N need not be a multiple of the 64-row tile.  The last, partial tile
 *     is read with every row index clamped to N-1, so no load leaves the
 *     tensors, and its missing keys are masked to -inf before the row max;
 *     rows past N are never written ("FlashAttention dataflow and
 *     engineering validation on MI50", §6.1: the boundary tile must be
 *     cropped and masked rather than read past the end; "CUDA
 *     FlashAttention ...", §5.4: ragged tails take masked loads).
 *   - Numerics: products on fp16/bf16 MFMA with FP32 accumulation; running
 *     max, sum and output accumulators in FP32 ("CUDA FlashAttention ...", §2);
 *     outputs rounded to the storage type with round-to-nearest-even.
 *
 * Error convention: every entry point returns FA_OK (0) or a positive
 * fa_status.  Argument errors are detected before anything is launched.
 * FA_ERR_HIP means a launch was rejected by the runtime; faults during
 * execution surface at the caller's next synchronisation of `stream`.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,       /* B, H or N <= 0, N > 2^30, H_kv not dividing H, or
                             the grid is too large                              */
  FA_ERR_UNSUPPORTED = 3, /* D, dtype, causal flag or scale unsupported          */
  FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                    */
  FA_ERR_WORKSPACE = 5,   /* backward workspace missing or smaller than needed   */
  FA_ERR_HIP = 6,         /* the HIP runtime rejected a launch                   */
  FA_ERR_SCRATCH_LIMIT = 7 /* fa_bwd_noalloc: the shape needs more workspace than
                              the library's static scratch holds                */
} fa_status;

typedef enum fa_dtype { FA_FP16 = 0, FA_BF16 = 1 } fa_dtype;

/*
 * fa_fwd -- attention forward.
 *   q, k, v : inputs [B,H,N,D] of `dtype`.
 *   o       : output [B,H,N,D] of `dtype`, O = softmax(scale*QK^T + M) V.
 *   lse     : output FP32 [B,H,N], natural-log log-sum-exp of each score row
 *             (with the mask applied).
 *   causal  : 0 = no mask, 1 = square top-left causal mask (key j visible to
 *             query i iff j <= i).  Tiles wholly above the diagonal are
 *             skipped ("Why FlashAttention ...", §4.5).
 *   scale   : multiplies Q K^T; callers pass 1/sqrt(D) for standard attention.
 * Returns FA_OK or an fa_status error code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t N, int64_t D,
           int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_kernel_name -- which forward kernel fa_fwd (and fa_fwd_ex with no
 * mask, dropout or split) runs for a launch of this shape (host-only, no GPU work; for profiling and tests).
 * All four compute the same online-softmax recurrence ("CUDA FlashAttention
 * ...", §4) and differ only in how the work is cut, so results agree up to
 * the order of floating-point additions:
 *   "fwd_short_kernel" -- fewer than 256 tiles of 128 queries (B*H*ceil(N/128),
 *       one per compute unit), or causal with exactly 256 and N >= 8192
 *       (there one workgroup would walk every key tile alone at the end):
 *       32 (D = 64) or 64 (D = 128) queries per
 *       workgroup with the keys split over its four waves and the partial
 *       states merged in LDS ("CUDA FlashAttention ...", §7, split along K);
 *   "fwd_short_pipe_kernel" -- the same split at D = 128 and N >= 1024, with
 *       a wave's two query blocks software-pipelined against each other;
 *   "fwd_d128_kernel" -- D = 128 with at least 1024 tiles of 256 queries:
 *       64 queries per wave, 256 per workgroup;
 *   "fwd_kernel" -- otherwise: 32 queries per wave, 128 per workgroup.
 * Returns a static string, "" for a shape fa_fwd would reject.
 */
const char* fa_fwd_kernel_name(int64_t B, int64_t H, int64_t N, int64_t D, int causal);

/*
 * fa_bwd_workspace_bytes -- bytes of device workspace fa_bwd needs: one FP32
 * value per query row for Delta_i = rowsum(dO_i * O_i), i.e. 4*B*H*N, rounded
 * up to 256; plus, when B*H*ceil(N/128) is too small to fill the GPU (few
 * heads of a long sequence), FP32 partial dK and dV as described for
 * fa_bwd_ex_workspace_bytes.  Returns 0 for arguments fa_bwd would reject.
 */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D,
                              int causal, int dtype);

/*
 * fa_bwd -- attention backward by recomputation.
 *   q, k, v, o, lse : the forward's inputs and outputs (o and lse exactly as
 *                     fa_fwd wrote them).
 *   dout            : upstream gradient dL/dO [B,H,N,D] of `dtype`.
 *   dq, dk, dv      : outputs [B,H,N,D] of `dtype`; fully overwritten.
 *   workspace       : device scratch of at least fa_bwd_workspace_bytes(...)
 *                     bytes, owned by the caller; its contents on entry are
 *                     ignored and on return are unspecified.
 *   other arguments : as for fa_fwd and with the same values.
 * Three kernels run in order on `stream`: Delta, then dK/dV (outer loop over
 * key tiles; with few heads, split into parts over the query tiles whose
 * FP32 partial sums a fourth kernel adds in a fixed order), then dQ (outer
 * loop over query tiles).  No atomics are used, so results are bitwise
 * reproducible.
 * Returns FA_OK or an fa_status error code.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout,
           void* dq, void* dk, void* dv,
           int64_t B, int64_t H, int64_t N, int64_t D,
           int causal, float scale, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, kernels and results as fa_bwd, with
 * the workspace taken from the library's own static device scratch of
 * FA_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends) instead of
 * a caller's buffer.  It allocates and frees nothing.
 *   Arguments : as for fa_bwd, without workspace and workspace_bytes.
 *   Limit     : shapes with fa_bwd_workspace_bytes(...) above
 *               FA_NOALLOC_SCRATCH_BYTES (e.g. more than 8M query rows B*H*N,
 *               or few heads of a long sequence, whose partial dK/dV sums
 *               need more) are rejected with FA_ERR_SCRATCH_LIMIT before any
 *               work is enqueued.
 *   Sharing   : every call on one GPU uses that GPU's one scratch array, so
 *               calls that overlap on one GPU (on different streams or from
 *               different threads) race; serialise them.  The scratch is the
 *               one of the GPU `stream` belongs to.
 * Returns FA_OK, FA_ERR_SCRATCH_LIMIT or another fa_status error code.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout,
                   void* dq, void* dk, void* dv,
                   int64_t B, int64_t H, int64_t N, int64_t D,
                   int causal, float scale, int dtype, void* stream);

/*
 * Key-padding masks (padded variable-length batches).
 *
 * A key-padding mask key_mask[B][N] (bytes, nonzero = visible) hides keys
 * of batch element b from every query of b, in every head, like the causal
 * mask: hidden scores are -inf before the row max.  A right-padded batch of
 * sequences with lengths L_b is key_mask[b][j] = (j < L_b).  A row left
 * with no visible key (possible with masks) gets O = 0 and LSE = -inf and
 * contributes nothing to any gradient.
 *
 * Block-level flags ("FlashAttention dataflow and engineering validation on
 * MI50", §4.3: on 64-wide waves the padding test belongs to the block loop,
 * once per block, not to every element): fa_mask_tiles compresses the byte
 * mask once into a tile table, which fa_fwd_ex and fa_bwd_ex read (through
 * fa_options.mask_tiles) instead of the mask.  They visit only tiles with a visible key, and test
 * elements only in tiles that are partly visible.
 *
 * Tile table (T = ceil(N/64); offsets from `tiles`, each section starting
 * on a 256-byte boundary):
 *   words  uint64 [B][T]    at 0: bit j of words[b][t] is set iff key
 *                           64t + j exists (< N) and is visible;
 *   prefix int32 [B][T+1]   at P = round_up(8*B*T, 256): number of tiles
 *                           before t with a nonzero word;
 *   list   int32 [B][T]     at P + round_up(4*B*(T+1), 256): list[b][i] is
 *                           the i-th tile with a nonzero word, ascending
 *                           (entries past prefix[b][T] unspecified).
 * A table serves every call with the same B and N (all heads, fwd and bwd).
 */

/* fa_mask_tiles_bytes -- size of the tile table for B, N; 0 if B, N are
 * out of range (B, N >= 1, N <= 2^30, B*ceil(N/64) < 2^31). */
size_t fa_mask_tiles_bytes(int64_t B, int64_t N);

/*
 * fa_mask_tiles -- build the tile table of key_mask (device, [B][N] bytes,
 * any alignment) into `tiles` (device, caller-owned, 16-byte aligned, at
 * least fa_mask_tiles_bytes(B, N) bytes) on `stream`.  Two kernels: one
 * wave per (b, tile) ballots the tile's 64 bytes into its word, then one
 * workgroup per b scans the words into prefix and list.
 * Errors: FA_ERR_NULL (key_mask), FA_ERR_SHAPE, FA_ERR_WORKSPACE (tiles
 * missing or short), FA_ERR_ALIGN, FA_ERR_HIP.
 */
int fa_mask_tiles(const uint8_t* key_mask, int64_t B, int64_t N, void* tiles, size_t tiles_bytes, void* stream);

/*
 * Attention dropout, regenerated instead of stored ("Why FlashAttention does
 * not need to store the attention matrix", §05: the kernel keeps only the
 * Philox seed and offset, and the backward pass rebuilds the same mask;
 * "CUDA FlashAttention ...", §7: the random offset must be reproducible).
 *
 * Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011), key
 * (seed, 0).  For batch element b, query head h, query i and key j the
 * counter is (j / 16, i, b*H + h, offset); the 256 output bits are 16
 * values of 16 bits, key j = 16t + e taking bits 16*(e % 4) .. +15 of word
 * e / 4.  Key j is kept for query i iff its value >= thr = floor(p * 65536);
 * kept probabilities are scaled by 65536 / (65536 - thr).  So:
 *   O = (P * Z * s) V, LSE is that of the undropped P, and the backward uses
 *   dV = (P*Z*s)^T dO, dS = P * ((dO V^T)*Z*s - Delta), Delta = rowsum(dO*O).
 * dropout_p must lie in [0, 1) (else FA_ERR_UNSUPPORTED); p = 0 keeps all.
 */

/*
 * fa_dropout_mask -- write the keep mask that dropout (fa_options) uses:
 * keep[b][h][i][j] = 1 (kept) or 0 (dropped), bytes, [B, H, N, N] on the
 * device (caller-owned, any alignment).  Meant for tests and inspection: it
 * is N*N bytes per head.  Errors: FA_ERR_NULL, FA_ERR_SHAPE (N > 2^24 or too
 * many threads), FA_ERR_UNSUPPORTED (p outside [0, 1)), FA_ERR_HIP.
 */
int fa_dropout_mask(uint8_t* keep, int64_t B, int64_t H, int64_t N,
                    float dropout_p, uint64_t seed, uint64_t offset, void* stream);

/*
 * Options of one call: the features beyond plain multi-head attention, set
 * in one struct instead of one entry point per combination.  Start from
 * FA_OPTIONS_DEFAULT (plain attention: fa_fwd / fa_bwd) and set the fields a
 * call uses; every combination is supported.  The backward of a forward
 * takes the same options (num_splits aside: the backward of a split forward
 * is the plain one).  A NULL options pointer means FA_OPTIONS_DEFAULT.
 *
 *   h_kv       : K/V heads (GQA; h_kv = 1 is MQA).  k, v (and dk, dv) are
 *                [B, h_kv, N, D]; query head h of batch element b reads K/V
 *                head h / (H / h_kv) of b in place, no copy ("CUDA
 *                FlashAttention ...", §7: query heads map onto a shared K/V
 *                head; the workgroups of one group are numbered onto the same
 *                XCD when B*h_kv is a multiple of 8).  The gradient of a shared
 *                K/V head is the sum over its H / h_kv query heads, added in
 *                FP32 registers (and, when the dK/dV pass runs in parts, by a
 *                reduce kernel in a fixed order): bitwise reproducible.
 *                0 means H.  FA_ERR_SHAPE if h_kv < 0 or does not divide H.
 *   mask_tiles : a key-padding mask as its tile table (fa_mask_tiles, same B
 *                and N; contents trusted), or NULL for none.  Hidden keys get
 *                dK = dV = 0 exactly; a row with no visible key gets O = 0,
 *                LSE = -inf and dQ = 0.  FA_ERR_ALIGN if not 16-byte aligned.
 *   dropout    : 1 = attention dropout with (dropout_p, dropout_seed,
 *                dropout_offset) as defined above (p = 0 keeps every
 *                probability but runs the dropout kernels); 0 = none.
 *                FA_ERR_UNSUPPORTED for another value or p outside [0, 1).
 *   num_splits : fa_fwd_ex only.  0 = one pass.  S in 1 .. 64: the keys are
 *                split into S contiguous ranges of whole 64-key tiles ("CUDA
 *                FlashAttention ...", §7: for long N and small B*H, split
 *                along K; each part yields a local (m, l, o), merged with the
 *                formula of §4).  Pass 1: one workgroup per (query tile,
 *                split) writes each row's split LSE_s and its output O_s
 *                normalised within the split (FP32, in the workspace; -inf
 *                for a split with no visible key).  Pass 2: LSE = m + ln
 *                sum_s exp(LSE_s - m), m = max_s LSE_s, and O = sum_s
 *                exp(LSE_s - LSE) O_s, rounded to dtype (RNE).  With dropout
 *                each split drops and scales its own probabilities and its
 *                partial LSE is that of the undropped ones, so the merge
 *                weights are unchanged; with a mask each split takes its
 *                share of the batch element's list of non-empty key tiles.
 *                FA_ERR_UNSUPPORTED outside 0 .. 64.
 */
typedef struct fa_options {
  int64_t h_kv;
  const void* mask_tiles;
  int dropout;
  float dropout_p;
  uint64_t dropout_seed;
  uint64_t dropout_offset;
  int num_splits;
} fa_options;

#define FA_OPTIONS_DEFAULT {0, NULL, 0, 0.0f, 0, 0, 0}

/*
 * fa_fwd_splitkv_num_splits -- a split count for the split-K/V forward
 * (fa_options.num_splits of fa_fwd_ex) on this
 * shape ("CUDA FlashAttention ...", §7: split along K when N is long and
 * B*H is small, so that there are enough workgroups).  The forward runs one
 * workgroup per 128 queries, W = B*H*ceil(N/128) of them; the count doubles,
 * from 1, while W*S < 512 (two workgroups per compute unit), each of the S
 * ranges would keep at least 2048 keys after the doubling, and S < 16.
 * Returns 1 when splitting would not pay (for example B=1 H=32 N=8192), and
 * 0 for a shape fa_fwd would reject.  Host-only: no GPU work.
 */
int fa_fwd_splitkv_num_splits(int64_t B, int64_t H, int64_t N, int64_t D, int causal);

/*
 * fa_fwd_ex_workspace_bytes -- bytes of device workspace fa_fwd_ex needs with
 * these options: for num_splits = S >= 1 an FP32 LSE and an FP32 D-vector per
 * query row and split, S*B*H*N*(D+1)*4 (each part rounded up to 256); 0 when
 * no workspace is needed (num_splits = 0) or for arguments fa_fwd_ex would
 * reject.  Host-only.
 */
size_t fa_fwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D,
                                 int causal, int dtype, const fa_options* opt);

/*
 * fa_fwd_ex -- fa_fwd with options (see fa_options).
 *   k, v      : [B, h_kv, N, D]; q, o : [B, H, N, D]; lse : FP32 [B, H, N].
 *   workspace : caller-owned device memory of at least
 *               fa_fwd_ex_workspace_bytes(...) bytes, 16-byte aligned (may be
 *               NULL when that is 0); contents on entry ignored, on return
 *               unspecified.
 * Other arguments, layouts and errors as for fa_fwd; additionally the option
 * errors above and FA_ERR_WORKSPACE for a missing or short workspace.
 * fa_fwd(...) is fa_fwd_ex(..., NULL, NULL, 0, stream).
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int64_t B, int64_t H, int64_t N, int64_t D,
              int causal, float scale, int dtype, const fa_options* opt,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_ex_workspace_bytes -- bytes of device workspace fa_bwd_ex needs:
 * Delta (4*B*H*N), plus, when the dK/dV pass splits the query positions of
 * each K/V head (its G = H / h_kv query heads' query tiles) into P > 1 parts
 * (few K/V heads: the pass would otherwise have too few workgroups to fill
 * the GPU; P is at most the larger of G and the number of 8-tile groups of
 * query tiles), FP32 partial dK and dV of 4*P*B*h_kv*N*D bytes each; and,
 * when the dQ pass runs in parts, FP32 partial dQ likewise; sections rounded
 * up to 256.  Equals fa_bwd_workspace_bytes for the default options; 0 for
 * arguments fa_bwd_ex would reject.  Host-only.
 */
size_t fa_bwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D,
                                 int causal, int dtype, const fa_options* opt);

/*
 * fa_bwd_ex -- fa_bwd for a forward computed by fa_fwd or fa_fwd_ex with the
 * same options (num_splits is ignored).  dk, dv : [B, h_kv, N, D]; every
 * other tensor as in fa_bwd.  Workspace: fa_bwd_ex_workspace_bytes(...).
 * Errors as for fa_bwd plus the option errors above.
 * fa_bwd(...) is fa_bwd_ex(..., NULL, workspace, workspace_bytes, stream).
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
              const float* lse, const void* dout,
              void* dq, void* dk, void* dv,
              int64_t B, int64_t H, int64_t N, int64_t D,
              int causal, float scale, int dtype, const fa_options* opt,
              void* workspace, size_t workspace_bytes, void* stream);

/* fa_status_str -- a static, human-readable name for a status code. */
const char* fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
