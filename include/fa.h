/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact-attention library (libfa.so).
 *
 * The operation is exact scaled-dot-product attention, O = softmax(scale * Q K^T) V,
 * computed as a tiled, IO-aware fused kernel: the N x N score matrix never reaches
 * HBM; the forward keeps a running row maximum m and a running sum of exponentials l
 * per query row and saves only O and the log-sum-exp ("ELI5: FlashAttention",
 * highlights on kernel fusion, tiling and the m(x)/l(x) statistics).  The backward
 * recomputes S and P from Q, K and the log-sum-exp ("ELI5: FlashAttention",
 * recomputation highlight) in one of the two designs compared in "Potential
 * algorithmic improvements for backward pass" (flash-attention issue 1172):
 *   - FA_BWD_5GEMM_ATOMIC: one dK/dV kernel that also accumulates dQ with fp32
 *     atomics (S, dP, dV, dK, dQ: five GEMMs; non-deterministic summation order);
 *   - FA_BWD_7GEMM: a dK/dV kernel (four GEMMs) followed by a separate dQ kernel
 *     that walks the keys in the forward's direction (three GEMMs); no atomics, so
 *     results are bitwise reproducible.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout     every tensor is contiguous [B, H, N, d] (d fastest), the statistics
 *             lse / delta are contiguous [B, H, N].  N_q == N_k == N.
 *  dtypes     q, k, v, dout: bfloat16 (raw 16-bit storage, passed as void*);
 *             o, lse, dq, dk, dv, delta: float32.
 *  Math       scale multiplies Q K^T; causal means query i attends to keys j <= i;
 *             lse is the natural-log log-sum-exp of the scaled, masked scores.
 *  Memory     every pointer is device memory allocated and owned by the caller; the
 *             library never allocates, frees or synchronises.  Pointers must be
 *             16-byte aligned.  Outputs may not alias inputs.
 *  Stream     all work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *             default stream) and is asynchronous: kernel faults surface at the
 *             caller's next synchronisation.
 *  Errors     arguments are validated before anything is enqueued; on any error
 *             nothing is launched and outputs are untouched.  FA_ERR_INVALID_ARG:
 *             null/misaligned pointer, B, H or N <= 0, non-finite or non-positive
 *             scale, aliasing, or a tensor too large for 32-bit in-head indexing;
 *             FA_ERR_UNSUPPORTED: head dim not in {64, 96, 128, 192, 256, 288, 320, 352,
 *             384} or unknown variant/config; FA_ERR_WORKSPACE: workspace missing or too small;
 *             FA_ERR_HIP: a launch failed (hipGetLastError after the launch);
 *             FA_ERR_TOO_LARGE: the problem exceeds the fixed scratch of
 *             fa_bwd_noalloc.
 *  Threads    stateless apart from a once-initialised device-property cache;
 *             safe to call from several host threads.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_WORKSPACE = 3,
  FA_ERR_HIP = 4,
  FA_ERR_TOO_LARGE = 5
} fa_status;

typedef enum {
  FA_BWD_5GEMM_ATOMIC = 0, /* dK/dV kernel with fused fp32-atomic dQ (5 GEMMs)          */
  FA_BWD_7GEMM = 1         /* dK/dV kernel, then a separate forward-direction dQ kernel */
} fa_bwd_variant;

/* Forward pass.
 * Computes o = softmax(scale * q k^T, causal mask) v and lse (natural log) per
 * query row ("ELI5: FlashAttention": tiling plus the online m/l statistics;
 * issue 1172, opening comment: the log-sum-exp is the saved operand).
 *   q, k, v : bf16 [B,H,N,d]          (read)
 *   o       : fp32 [B,H,N,d]          (written)
 *   lse     : fp32 [B,H,N]            (written)
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, int B, int H, int N, int d, int causal,
                 float scale, float* o, float* lse, void* stream);

/* Bytes of workspace fa_bwd needs: the fp32 row term delta_i = sum_k dO_ik O_ik,
 * [B,H,N] floats, for either variant.  Returns 0 for invalid sizes. */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, fa_bwd_variant variant);

/* Backward pass: gradients of L = sum(dout * o) with respect to q, k, v.
 * Recomputes S and P from q, k and lse (issue 1172: recomputation instead of
 * storing P; "ELI5: FlashAttention", recomputation highlight), in the chosen
 * design (see the top of this file).  causal and scale must equal the forward's.
 *   q, k, v, dout : bf16 [B,H,N,d]    (read)
 *   o, lse        : fp32, as written by fa_fwd (read)
 *   dq, dk, dv    : fp32 [B,H,N,d]    (written; dq is zeroed by the library first
 *                                      for the atomic variant)
 *   workspace     : >= fa_bwd_workspace_size bytes of device memory, 16-B aligned
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
                 const void* dout, int B, int H, int N, int d, int causal, float scale,
                 fa_bwd_variant variant, float* dq, float* dk, float* dv, void* workspace,
                 size_t workspace_bytes, void* stream);

/* fa_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, semantics and kernels as fa_bwd; the backward's one scratch buffer,
 * the fp32 row term delta [B,H,N], is a fixed array inside the library of
 * FA_NOALLOC_MAX_ROWS floats (32 MiB) on each GPU it runs on, held until the process
 * ends.  The array's address is looked up once per device, on the first call with that
 * device current.  B*H*N above FA_NOALLOC_MAX_ROWS returns FA_ERR_TOO_LARGE before
 * anything is enqueued.  The library allocates, frees and synchronises nothing.  All
 * calls on one GPU share its array: calls whose work overlaps on one GPU (concurrent
 * streams, host threads) race and must be serialised by the caller; each call writes
 * every row of delta it later reads, so nothing needs clearing between calls. */
#define FA_NOALLOC_MAX_ROWS (1u << 23)
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const float* o, const float* lse,
                         const void* dout, int B, int H, int N, int d, int causal, float scale,
                         fa_bwd_variant variant, float* dq, float* dk, float* dv, void* stream);

/* The backward's first step on its own: delta_i = sum_k dout_ik * o_ik per row
 * (the softmax-backward row term, computed from O instead of from P and dP; the
 * two are equal because O = P V and dP = dO V^T).  When zero_dq is non-zero it
 * also writes zeros to dq (the atomic variant's accumulator).
 *   o : fp32 [B,H,N,d], dout : bf16 [B,H,N,d], delta : fp32 [B,H,N], dq : fp32 or NULL */
fa_status fa_bwd_preprocess(const float* o, const void* dout, int B, int H, int N, int d, float* delta,
                            float* dq, int zero_dq, void* stream);

/* The backward's kernel stages on their own.  fa_bwd runs, for the 5-GEMM design,
 * fa_bwd_preprocess (with zero_dq) and then fa_bwd_dkdv with atomic_dq; for the 7-GEMM
 * design, fa_bwd_dq_delta and then fa_bwd_dkdv.  For fa_bwd_dkdv and fa_bwd_dq, delta
 * must hold the preprocess result for the same o/dout.
 * fa_bwd_dkdv: dk, dv (fp32 [B,H,N,d], written).  With atomic_dq != 0 it also adds
 *   scale * dS K into dq with fp32 atomics (the 5-GEMM design; dq must already be
 *   zero or hold a partial sum); with atomic_dq == 0, dq is ignored (may be NULL).
 * fa_bwd_dq: the 7-GEMM design's dQ kernel; dq (fp32 [B,H,N,d]) is written once per
 *   element, no atomics.
 * cfg: tile configuration index (-1 = default) of pass 1/2 (dkdv) or 3 (dq). */
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                      const float* delta, int B, int H, int N, int d, int causal, float scale, int atomic_dq,
                      float* dq, float* dk, float* dv, void* stream, int cfg);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                    const float* delta, int B, int H, int N, int d, int causal, float scale, float* dq,
                    void* stream, int cfg);

/* The 7-GEMM design's first backward launch: the dQ kernel computing each row's delta
 * itself (the preprocess's sum_k dout_ik * o_ik, from the dO rows the kernel loads for
 * its own products and the same columns of o) instead of reading it, and writing it to
 * delta for fa_bwd_dkdv, which runs after it -- one launch and one pass over O and dO
 * fewer than preprocess + dQ.
 *   o : fp32 [B,H,N,d] (read), delta : fp32 [B,H,N] (written), dq : fp32 [B,H,N,d]
 *   (written once per element); delta must overlap neither o, dq nor lse.
 * Errors as fa_bwd_dq; cfg: tile configuration of pass 3 (-1 = default). */
fa_status fa_bwd_dq_delta(const void* q, const void* k, const void* v, const float* o, const void* dout,
                          const float* lse, int B, int H, int N, int d, int causal, float scale, float* delta,
                          float* dq, void* stream, int cfg);

/* Tile configurations, for the block-shape sweep ("Potential algorithmic
 * improvements for backward pass": search over block dimensions under register
 * pressure; non-square blocks such as 32-64 x 160-320).
 * pass: 0 = forward, 1 = backward dK/dV (7-GEMM), 2 = backward dK/dV with atomic dQ,
 *       3 = backward dQ (7-GEMM).
 * fa_num_configs returns how many configurations exist for (pass, d, causal);
 * fa_config_name writes a NUL-terminated description of config `index` into buf
 * (rows per workgroup x keys/queries per tile, waves) and returns 0, or -1 if out
 * of range.  fa_default_config returns the index the plain entry points use. */
int fa_num_configs(int pass, int d, int causal);
int fa_config_name(int pass, int d, int causal, int index, char* buf, size_t buf_len);
int fa_default_config(int pass, int d, int causal);

/* fa_fwd / fa_bwd with explicit tile configurations (-1 = default).  For fa_bwd_ex,
 * cfg_dkdv indexes pass 1 or 2 according to the variant, cfg_dq indexes pass 3
 * (ignored by the atomic variant). */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, int B, int H, int N, int d, int causal,
                    float scale, float* o, float* lse, void* stream, int cfg);
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse,
                    const void* dout, int B, int H, int N, int d, int causal, float scale,
                    fa_bwd_variant variant, float* dq, float* dk, float* dv, void* workspace,
                    size_t workspace_bytes, void* stream, int cfg_dkdv, int cfg_dq);

/* ---------------------------------------------------------------------------
 * General entry points: any head dimension 1 <= d <= 384 and strided views.
 *
 * Every [B,H,N,d] tensor is described by its base pointer and element strides
 * (b, h, n): element (b, h, n, i) is at base[b*stride.b + h*stride.h + n*stride.n + i]
 * (the head dimension is contiguous; strides are >= 0).  lse stays contiguous
 * [B,H,N].  Pointers need only element alignment (2 bytes for bf16, 4 for fp32;
 * lse 16 bytes).  The math is that of fa_fwd / fa_bwd; the pages' kernels are
 * built for fixed head dimensions, and issue 1172 asks for arbitrary head
 * dimensions with strided rows.  The fused kernels run at Dp = the smallest of 64,
 * 96, 128, 192, 256 that is >= d, or above 256 d rounded up to a multiple of 32, with columns d .. Dp-1 taken as zeros (zero columns change
 * no score, so the result is the attention of the d columns):
 *   - in place, reading and writing the caller's views directly, when d is a
 *     multiple of 8, every base pointer is 16-byte aligned, every stride is a
 *     multiple of 16 bytes, q and dout share their row stride, and N * stride.n
 *     stays below 2^31 bytes per view; the kernels pad the head dim themselves and
 *     touch no element past column d.  The backward then needs the row-term
 *     workspace of fa_bwd at Dp, plus a [B,H,N,Dp] fp32 dq accumulator for the
 *     5-GEMM variant unless dq is contiguous with d == Dp;
 *   - otherwise through zero-padded contiguous copies held in the workspace,
 *     whose results' first d columns are written into the caller's views.
 * Validation and errors as above; views that overlap an output are rejected
 * (FA_ERR_INVALID_ARG), d outside 1..384 is FA_ERR_UNSUPPORTED (with dropout, d above
 * 256 as well). */
typedef struct {
  long long b, h, n;
} fa_strides;

/* Workspace bytes of the padded path (an upper bound for every call with these sizes). */
size_t fa_fwd_general_workspace_size(int B, int H, int N, int d);
size_t fa_bwd_general_workspace_size(int B, int H, int N, int d, fa_bwd_variant variant);

/* Forward: q, k, v bf16 views; o fp32 view (written); lse fp32 [B,H,N] (written). */
fa_status fa_fwd_general(const void* q, fa_strides q_str, const void* k, fa_strides k_str, const void* v,
                         fa_strides v_str, int B, int H, int N, int d, int causal, float scale, float* o,
                         fa_strides o_str, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Backward: q, k, v, dout bf16 views and o fp32 view (read), lse fp32 [B,H,N] (read);
 * dq, dk, dv fp32 views (written). */
fa_status fa_bwd_general(const void* q, fa_strides q_str, const void* k, fa_strides k_str, const void* v,
                         fa_strides v_str, const float* o, fa_strides o_str, const float* lse, const void* dout,
                         fa_strides dout_str, int B, int H, int N, int d, int causal, float scale,
                         fa_bwd_variant variant, float* dq, fa_strides dq_str, float* dk, fa_strides dk_str,
                         float* dv, fa_strides dv_str, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Dropout on the attention probabilities, fused into the kernels.
 *
 * Dropout is one of the elementwise passes over the N x N matrix that unfused
 * attention spends its time on ("ELI5: FlashAttention", standard-attention
 * highlights); here it runs inside the fused kernels and its mask never reaches
 * memory.  The pages fix no random-number generator; this library draws the keep
 * decision of element (b, h, i, j) (query i, key j) from Philox4x32-10 (Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC '11):
 *   key      (seed & 0xffffffff, seed >> 32)
 *   counter  (j / 8, i, b * H + h, offset)
 *   draw     16-bit half (j % 2) of output word (j % 8) / 2, low half first
 *   keep     draw >= t, t = floor(p * 65536) capped at 65535
 * so the drop probability is t / 65536 (p rounded down to a multiple of 2^-16);
 * kept probabilities are scaled by 65536 / (65536 - t), the reciprocal of the keep
 * probability (fa_dropout_keep_scale), so E[o] is the undropped output.
 * The forward computes o = (P * M * s) v with lse that of the undropped scores;
 * the backward gives the gradients of sum(dout * o) for that same mask, redrawn
 * from (seed, offset): pass the forward's values.  A p that rounds to t = 0 runs the
 * plain kernels.  Head dims 64, 96, 128, 192, 256 here (any d in 1..256 through the general
 * dropout entries below; above 256 dropout is FA_ERR_UNSUPPORTED); each pass runs one tile
 * shape per head dim.
 * Errors as above; p outside [0, 1) or not finite is FA_ERR_INVALID_ARG. */
typedef struct {
  double p;                /* drop probability, 0 <= p < 1                           */
  unsigned long long seed; /* generator key                                          */
  unsigned offset;         /* fourth counter word (e.g. a step or layer index)       */
} fa_dropout;
/* Forward with dropout: arguments and outputs as fa_fwd. */
fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, int B, int H, int N, int d, int causal,
                         float scale, fa_dropout dropout, float* o, float* lse, void* stream);
/* Backward with dropout: arguments, outputs and workspace as fa_bwd; o and lse are the
 * dropout forward's, dropout must equal the forward's. */
fa_status fa_bwd_dropout(const void* q, const void* k, const void* v, const float* o, const float* lse,
                         const void* dout, int B, int H, int N, int d, int causal, float scale, fa_dropout dropout,
                         fa_bwd_variant variant, float* dq, float* dk, float* dv, void* workspace,
                         size_t workspace_bytes, void* stream);
/* The factor kept probabilities are scaled by for drop probability p: 65536 / (65536 - t);
 * -1 if p is outside [0, 1). */
double fa_dropout_keep_scale(double p);
/* Dropout through the general entry points (any d in 1..256, strided views): arguments,
 * workspace and errors as fa_fwd_general / fa_bwd_general.  The keep decisions depend on
 * (b, h, i, j) only, so they are the same as those of fa_fwd_dropout for the same seed,
 * offset and sequence positions. */
fa_status fa_fwd_general_dropout(const void* q, fa_strides q_str, const void* k, fa_strides k_str, const void* v,
                                 fa_strides v_str, int B, int H, int N, int d, int causal, float scale,
                                 fa_dropout dropout, float* o, fa_strides o_str, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);
fa_status fa_bwd_general_dropout(const void* q, fa_strides q_str, const void* k, fa_strides k_str, const void* v,
                                 fa_strides v_str, const float* o, fa_strides o_str, const float* lse,
                                 const void* dout, fa_strides dout_str, int B, int H, int N, int d, int causal,
                                 float scale, fa_dropout dropout, fa_bwd_variant variant, float* dq,
                                 fa_strides dq_str, float* dk, fa_strides dk_str, float* dv, fa_strides dv_str,
                                 void* workspace, size_t workspace_bytes, void* stream);
/* Human-readable name of a status code (static storage). */
const char* fa_status_string(fa_status s);

/* Library version string, e.g. "fa-mi355x 0.1 gfx950". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
