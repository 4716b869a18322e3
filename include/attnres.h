/*
 * attnres.h - C ABI of the MI355X (gfx950) decode-step hot path:
 * a weight-stationary skinny GEMM (the attention output projection) fused
 * with the post-projection AttnRes epilogue.
 *
 * The operations are the ones the vLLM API pages of the Kimi-K3 specialized
 * decode (CuTe DSL modules) describe:
 *   - gemm.ws_gemm page, WsGemm (module summary: y[M, N] = x[M, K] W[N, K]^T,
 *     BF16 operands, FP32 accumulation, the K parts summed in K order) and
 *     positive_zero (a -0.0 result is stored as +0.0);
 *   - attn_res.kernel page, ClusterAttnRes (module summary; methods pre,
 *     weights, post; helper rstd): AttnRes for one token;
 *   - oproj.prepared page, module summary and PreparedOproj.run: the
 *     o-projection output is the AttnRes delta of the same layer; prefix and
 *     saved blocks are updated in place.
 *
 * Conventions shared by every entry point
 *   - bfloat16 tensors are passed as raw 16-bit patterns (uint16_t).
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     allocates nothing and keeps no state between calls.
 *   - Strides (ld_*, blk_stride_*) count elements, not bytes. Rows are
 *     contiguous. Every tensor pointer must be 16-byte aligned and every
 *     stride a multiple of 8 elements (16-byte vector loads and stores).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work: they return before the GPU has finished and
 *     never synchronise the host.
 *   - All arguments are checked on the host before anything is enqueued; an
 *     invalid call returns a negative code and touches no memory.
 *   - No argument may alias another, except as stated (prefix and blocks are
 *     read and written by the same call).
 *   - Rows past T (or M) and block slots other than `write` are never written.
 *   - NaN or infinite inputs give unspecified outputs.
 *   - Calls on one stream are ordered; calls that run concurrently on different
 *     streams must not share output tensors or a workspace.
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ATTNRES_OK 0
#define ATTNRES_EINVAL (-1)       /* null pointer, negative or inconsistent size or stride */
#define ATTNRES_EALIGN (-2)       /* pointer not 16-byte aligned or stride not a multiple of 8 */
#define ATTNRES_ERANGE (-3)       /* nb, write, cap, M or T outside the supported range */
#define ATTNRES_EUNSUPPORTED (-4) /* shape the kernels do not cover (H, N, K limits below) */
#define ATTNRES_EWORKSPACE (-5)   /* workspace missing, too small or misaligned */
#define ATTNRES_EHIP (-6)         /* the HIP runtime refused the launch */

/* Limits. */
#define ATTNRES_MAX_BLOCKS 8 /* saved blocks scored per token (nb) */
#define ATTNRES_MAX_M 64     /* tokens per GEMM or fused call */
#define ATTNRES_MAX_H 8192   /* hidden width of the AttnRes paths */

/*
 * attnres_run - AttnRes of T tokens with the delta given as a tensor
 * (attn_res.kernel page: ClusterAttnRes with a tensor delta, methods pre and
 * post). For every token t < T, with H the hidden width:
 *
 *   w      = norm * query                                     (weights)
 *   r(s,e) = 1 / sqrt(s / H + e)                              (rstd)
 *   l_b    = (blocks[t,b] . w) * r(sum blocks[t,b]^2, eps)    b < nb
 *   new    = bf16(prefix[t] + delta[t])  if has_delta,
 *            delta[t]                    otherwise (prefix is then not read)
 *   l_n    = (new . w) * r(sum new^2, eps)
 *   p      = softmax(l_0, ..., l_{nb-1}, l_n)
 *   h      = sum_b p_b blocks[t,b] + p_n new  (h = new when nb == 0),
 *            rounded to bf16 when final_boundary != 0
 *   out[t] = bf16(h * r(sum h^2, out_eps) * out_norm)
 *   prefix[t] <- new; aux[t] <- new (aux != NULL);
 *   blocks[t, write] <- new (write >= 0).
 * Saved blocks are scored with their values at launch, so write may name a
 * scored slot. bf16() rounds to nearest, ties to even.
 *
 * Arguments (bf16 unless stated):
 *   delta     [T, H], row stride ld_delta                        (read)
 *   prefix    [T, H], row stride ld_prefix                       (read if has_delta, written)
 *   blocks    [T, cap, H], element (t, b, i) at
 *             t*blk_stride_t + b*blk_stride_b + i; may be NULL when nb == 0 and write == -1
 *   norm, query, out_norm   [H]                                  (read)
 *   out       [T, H], row stride ld_out                          (written)
 *   aux       [T, H], row stride ld_aux, or NULL                 (written)
 *   eps       epsilon of the scoring RMSNorm (every logit)
 *   out_eps   epsilon of the output RMSNorm
 *   T >= 0 tokens (T == 0 returns ATTNRES_OK at once, whatever the other
 *   arguments); 8 <= H <= 8192, H % 8 == 0;
 *   0 <= nb <= min(8, cap); write == -1 or 0 <= write < cap;
 *   has_delta, final_boundary: 0 or 1.
 * Saved-block rows must not overlap: blk_stride_b >= H and blk_stride_t >= H,
 * and either blk_stride_t >= cap*blk_stride_b or blk_stride_b >= T*blk_stride_t.
 */
int attnres_run(const void* delta, int64_t ld_delta, void* prefix, int64_t ld_prefix,
                void* blocks, int64_t blk_stride_t, int64_t blk_stride_b, int cap,
                const void* norm, const void* query, const void* out_norm, void* out,
                int64_t ld_out, void* aux, int64_t ld_aux, float eps, float out_eps, int T,
                int H, int nb, int write, int has_delta, int final_boundary, void* stream);

/*
 * wsgemm_run - weight-stationary skinny GEMM (gemm.ws_gemm page, WsGemm):
 *   y[m, n] = bf16( sum_k x[m, k] W[n, k] )  for m < M, n < N,
 * FP32 accumulation over K, one rounding to bf16 (nearest even), and a -0.0
 * result stored as +0.0 (positive_zero). The K partial sums are added in a
 * fixed order, so results are bitwise reproducible run to run.
 *   x [M, K] row stride ldx; W [N, K] row stride ldw; y [M, N] row stride ldy.
 *   0 <= M <= 64 (M == 0 returns ATTNRES_OK at once); N >= 8, N % 8 == 0;
 *   K >= 0, K % 8 == 0. K == 0 gives y = +0.0; x, W, ldx and ldw are then
 *   not used and may be NULL / 0.
 */
int wsgemm_run(const void* x, int64_t ldx, const void* W, int64_t ldw, void* y, int64_t ldy,
               int M, int N, int K, void* stream);

/*
 * attnres_oproj_workspace_size - bytes of device workspace attnres_oproj_run
 * needs for M tokens and hidden width H (nb does not change it): a 256-byte
 * header and one bf16 mailbox row per token.
 */
size_t attnres_oproj_workspace_size(int M, int H, int nb);

/*
 * attnres_oproj_workspace_init - prepares a workspace once, after allocation:
 * zeroes the header and arms every mailbox word (enqueued on `stream`).
 * Every attnres_oproj_run call leaves the workspace armed again. The first
 * 32-bit word of the header becomes nonzero if a call ever gave up waiting
 * for its own workgroups (a safety bound of about a second per wait that a
 * healthy device never reaches); that call's outputs are then invalid.
 *   workspace: device memory, 256-byte aligned; bytes: a multiple of 4, at
 *   least 256.
 */
int attnres_oproj_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * attnres_oproj_run - the fused decode step: the o-projection of x (the
 * attention output, [M, K]) by W ([H, K]) gives the delta of AttnRes
 * (oproj.prepared page, module summary and PreparedOproj.run):
 *   delta = wsgemm(x, W)   (bf16, -0.0 stored as +0.0; never written to memory)
 * followed by attnres_run on that delta with T = M. All AttnRes arguments mean
 * what they mean for attnres_run.
 *   x [M, K] row stride ldx; W [H, K] row stride ldw; 1 <= M <= 64;
 *   K >= 0, K % 8 == 0 (K == 0: delta = +0.0, x and W unused and may be NULL);
 *   H as for attnres_run.
 *   workspace: at least attnres_oproj_workspace_size(M, H, nb) bytes, 256-byte
 *   aligned, prepared once by attnres_oproj_workspace_init; calls that may run
 *   at the same time need distinct workspaces.
 */
int attnres_oproj_run(const void* x, int64_t ldx, const void* W, int64_t ldw, int K, void* prefix,
                      int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                      int64_t blk_stride_b, int cap, const void* norm, const void* query,
                      const void* out_norm, void* out, int64_t ld_out, void* aux, int64_t ld_aux,
                      float eps, float out_eps, int M, int H, int nb, int write, int has_delta,
                      int final_boundary, void* workspace, size_t workspace_bytes, void* stream);

/* attnres_strerror - a static, human-readable description of a return code. */
const char* attnres_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
