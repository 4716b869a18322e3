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
#define ATTNRES_EWAIT (-7)        /* a wait of an earlier call on the workspace gave up */

/* Limits. */
#define ATTNRES_MAX_BLOCKS 8 /* saved blocks scored per token (nb) */
#define ATTNRES_MAX_M 64     /* tokens per GEMM or fused call */
#define ATTNRES_MAX_M_WS 128 /* tokens per wsgemm_run_ws call */
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
 * wsgemm_moe_front_run - wsgemm_run with WsGemm's MoE-front epilogue
 * (gemm.ws_gemm page: module summary and WsGemm.epilogue): the N output rows
 * of y = x W^T are a router shard, padding and a latent shard, written into
 * out [M, ld_out] (bf16 patterns; the pages' [capacity, width] mailbox rows):
 *   c <  valid          : the FP32 word of y[m, c] (FP32 accumulation, -0.0
 *                         stored as +0.0) at bf16 columns
 *                         router_base + 2 (slot + c) and + 1 (low half first);
 *   valid <= c < split  : not written (padding);
 *   c >= split          : bf16(y[m, c]) (-0.0 -> +0.0) at column base + c - split.
 * Nothing else in out is written.
 *   x [M, K], W [N, K] as for wsgemm_run (0 <= M <= 64, N % 8 == 0, K % 8 == 0);
 *   out: 16-byte aligned, ld_out a multiple of 8 (any width, may be < N);
 *   0 <= valid <= split <= N, valid and split multiples of 8; router_base and
 *   base even and >= 0, slot >= 0; router_base + 2 (slot + valid) <= ld_out
 *   when valid > 0 and base + N - split <= ld_out when split < N; the two
 *   shards' column ranges must not overlap.
 * Errors: those of wsgemm_run; ATTNRES_ERANGE for offsets outside the row,
 * ATTNRES_EALIGN for valid / split / router_base / base off their multiples.
 */
int wsgemm_moe_front_run(const void* x, int64_t ldx, const void* W, int64_t ldw, void* out,
                         int64_t ld_out, int M, int N, int K, int router_base, int slot, int base,
                         int valid, int split, void* stream);

/*
 * wsgemm_workspace_size - bytes of device workspace wsgemm_run_ws needs for M
 * tokens and N rows: a 256-byte header and, beyond 32 tokens, the hand-off of
 * FP32 partial products between the workgroups that split K.
 */
size_t wsgemm_workspace_size(int M, int N);

/*
 * wsgemm_run_ws - wsgemm_run (same arguments, same result up to the order of
 * the FP32 partial sums) with a caller workspace, which lets the call split K
 * across workgroups beyond 32 tokens (gemm.ws_gemm page, module summary: a
 * cluster of CTAs splits K and sums the parts in K order; here up to four
 * workgroups per 64-row group, the parts added in K order by the last one).
 * The sums are still in a fixed order: results are bitwise reproducible run
 * to run. Up to 32 tokens it runs wsgemm_run's kernel (bit for bit). It takes
 * up to ATTNRES_MAX_M_WS tokens in one pass over W (the pages stream token
 * groups for the same purpose); beyond 64 tokens the split is required:
 * K >= 256 and 2 * ceil(N / 64) <= the device's compute units, else
 * ATTNRES_EUNSUPPORTED.
 *   workspace: at least wsgemm_workspace_size(M, N) bytes, 256-byte aligned,
 *   prepared once by attnres_oproj_workspace_init (the same format); every
 *   call leaves it prepared again. If a wait gave up (the safety bound of
 *   attnres_oproj_run) the workspace stays flagged as described there
 *   (attnres_workspace_status). Calls that may run at the same time need
 *   distinct workspaces.
 * Errors: those of wsgemm_run, and ATTNRES_EWORKSPACE.
 */
int wsgemm_run_ws(const void* x, int64_t ldx, const void* W, int64_t ldw, void* y, int64_t ldy,
                  int M, int N, int K, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attnres_oproj_workspace_size - bytes of device workspace attnres_oproj_run
 * needs for M tokens and hidden width H (nb does not change it): a 256-byte
 * header, one bf16 mailbox row per token and, beyond 32 tokens, one FP32 row
 * per token (token count rounded up to a multiple of 16): the partial products
 * that one of the two workgroups splitting K hands to the other.
 */
size_t attnres_oproj_workspace_size(int M, int H, int nb);

/*
 * attnres_oproj_workspace_init - prepares a workspace once, after allocation:
 * zeroes the header and arms every mailbox word (enqueued on `stream`).
 * Every attnres_oproj_run call leaves the workspace armed again. The first
 * 32-bit word of the header becomes nonzero if a call ever gave up waiting
 * for its own workgroups (a safety bound of about a second per wait that a
 * healthy device never reaches). That call's outputs are then invalid, and
 * every later call on the flagged workspace is accepted but writes nothing
 * at all, until this call prepares the workspace again;
 * attnres_workspace_status reports the flag.
 *   workspace: device memory, 256-byte aligned; bytes: a multiple of 4, at
 *   least 256.
 */
int attnres_oproj_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * attnres_workspace_status - whether a wait of a call on this workspace
 * (attnres_oproj_run and its prepared-W and look-ahead forms, wsgemm_run_ws) gave up: waits
 * until the work enqueued on `stream` so far has finished (it synchronises
 * the host with the stream; not for use under stream capture), then reads the
 * workspace header. workspace == NULL with workspace_bytes == 0 names the
 * current device's array of attnres_oproj_run_noalloc (ATTNRES_OK if no call
 * has used it).
 * Returns ATTNRES_OK (no wait gave up: the outputs of every call so far are
 * valid), ATTNRES_EWAIT (a wait gave up: see attnres_oproj_workspace_init),
 * ATTNRES_EWORKSPACE (NULL, fewer than 256 bytes or not 256-byte aligned) or
 * ATTNRES_EHIP (the copy or the synchronisation failed).
 */
int attnres_workspace_status(const void* workspace, size_t workspace_bytes, void* stream);

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

/*
 * attnres_packed_weights_size - bytes of the prepared (tile-major) layout of
 * a W [N, K] for attnres_oproj_packed_run: 256 * N * 4 * ceil(K / 512).
 */
size_t attnres_packed_weights_size(int N, int K);

/*
 * attnres_pack_weights - writes W [N, K] (bf16, row stride ldw) once in the
 * prepared layout that attnres_oproj_packed_run streams (oproj.prepared page,
 * PreparedOproj.__init__: the projection weight is bound once, when the layer
 * is prepared, not per step). Layout: P = 4 * ceil(K / 512) planes of 128
 * k-values; plane j holds every row's k-values [128 j, 128 j + 128) as one
 * 256-byte segment, rows in order (segment of row n at byte (j N + n) * 256),
 * and inside the segment of row n the 16-byte piece p (k-values 8p .. 8p + 7
 * of the plane) sits at position p ^ (n & 15); k-values at or past K are
 * zero. The step then reads each plane front to back in whole segments of
 * consecutive rows, and the pieces land in LDS in the order its matrix-core
 * reads expect.
 *   W: device memory, 16-byte aligned, ldw >= K, a multiple of 8; K % 8 == 0;
 *   Wp: device memory of at least attnres_packed_weights_size(N, K) bytes,
 *   16-byte aligned, not overlapping W (written completely).
 *   N == 0 or K == 0 returns ATTNRES_OK at once.
 * Errors: ATTNRES_EINVAL (NULL, ldw < K, Wp too small), ATTNRES_EALIGN,
 * ATTNRES_EUNSUPPORTED (K % 8 != 0), ATTNRES_EHIP.
 */
int attnres_pack_weights(const void* W, int64_t ldw, int N, int K, void* Wp, size_t Wp_bytes,
                         void* stream);

/*
 * attnres_oproj_packed_run - attnres_oproj_run with W given in the prepared
 * layout (attnres_pack_weights of W [H, K]; Wp_bytes at least
 * attnres_packed_weights_size(H, K)). Up to 32 tokens it is the same
 * arithmetic in the same order: the outputs equal attnres_oproj_run's on the
 * row-major W bit for bit. Beyond 32 tokens, where two workgroups split K,
 * each workgroup takes its chunks of a prepared W in K order (all of them
 * sweep the planes together), while attnres_oproj_run starts each workgroup
 * at a different chunk (workgroups sharing x then read different parts of it
 * at a time): the FP32 sums then differ by rounding only.
 * Arguments and errors as for attnres_oproj_run (ldw is not needed); a
 * prepared W of 2^32 bytes or more returns ATTNRES_EUNSUPPORTED.
 */
int attnres_oproj_packed_run(const void* x, int64_t ldx, const void* Wp, size_t Wp_bytes, int K,
                             void* prefix, int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                             int64_t blk_stride_b, int cap, const void* norm, const void* query,
                             const void* out_norm, void* out, int64_t ld_out, void* aux,
                             int64_t ld_aux, float eps, float out_eps, int M, int H, int nb,
                             int write, int has_delta, int final_boundary, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * attnres_oproj_run_noalloc - attnres_oproj_run without a caller workspace,
 * for callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation). It allocates
 * nothing: its workspace is a device array inside the library, one per
 * device, ATTNRES_NOALLOC_WORKSPACE_BYTES (the largest workspace
 * attnres_oproj_run needs: 64 tokens of 8192 columns), held until the
 * process ends. The first call on a device looks the array up and enqueues
 * one small kernel that arms it, ahead of the step on `stream`. Every
 * argument means what it means for attnres_oproj_run, which gives the same
 * bits; sizes beyond the array (none within the limits of attnres_oproj_run)
 * return ATTNRES_EWORKSPACE.
 * Every call on a device shares that device's array, which each call leaves
 * armed for the next: calls that may overlap on one device (other streams,
 * other threads, graph replays running beside eager calls) race and must be
 * ordered by the caller. `stream` must belong to the current device
 * (ATTNRES_EINVAL otherwise). attnres_workspace_status(NULL, 0, stream)
 * reports whether a wait of a call on the current device's array gave up;
 * the array then stays flagged (later calls write nothing) until the process
 * ends.
 */
#define ATTNRES_NOALLOC_WORKSPACE_BYTES 3145984
int attnres_oproj_run_noalloc(const void* x, int64_t ldx, const void* W, int64_t ldw, int K,
                              void* prefix, int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                              int64_t blk_stride_b, int cap, const void* norm, const void* query,
                              const void* out_norm, void* out, int64_t ld_out, void* aux,
                              int64_t ld_aux, float eps, float out_eps, int M, int H, int nb,
                              int write, int has_delta, int final_boundary, void* stream);

/*
 * attnres_oproj_ahead_run - attnres_oproj_run that also stores the saved-block
 * statistics of the next layer's AttnRes over the same saved blocks
 * (oproj.prepared page: PreparedOproj.bind_ahead, and compile_oproj's `ahead`
 * rows; the statistics are the state ClusterAttnRes carries from pre to post
 * on the attn_res.kernel page: the mixture row and maximum / exp_sum). With
 * w' = next_norm * next_query and, for b < nb, the saved blocks as they are at
 * launch (a scored slot that this call overwrites contributes its old value):
 *   l'_b        = (blocks[t,b] . w') * r(sum blocks[t,b]^2, next_eps)
 *   scal[t]     = (m, S):  m = max_b l'_b,  S = sum_b exp(l'_b - m)
 *   mixture[t]  = sum_b exp(l'_b - m) blocks[t,b]
 * in FP32 (nb == 0: m = S = 0 and mixture[t] = 0). Every other argument and
 * every other output are those of attnres_oproj_run, bit for bit.
 *   next_norm, next_query [H] bf16 (read); next_eps >= 0.
 *   mixture [M, H] FP32, row stride ld_mixture >= H, a multiple of 8 (written);
 *   scal [M, 2] FP32, 8-byte aligned (written). They must not alias any other
 *   argument.
 * Errors: those of attnres_oproj_run, and ATTNRES_EINVAL / ATTNRES_EALIGN for
 * the arguments above.
 */
int attnres_oproj_ahead_run(const void* x, int64_t ldx, const void* W, int64_t ldw, int K,
                            void* prefix, int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                            int64_t blk_stride_b, int cap, const void* norm, const void* query,
                            const void* out_norm, void* out, int64_t ld_out, void* aux,
                            int64_t ld_aux, float eps, float out_eps, int M, int H, int nb,
                            int write, int has_delta, int final_boundary,
                            const void* next_norm, const void* next_query, float next_eps,
                            float* mixture, int64_t ld_mixture, float* scal, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * attnres_oproj_packed_ahead_run - attnres_oproj_ahead_run with W given in the
 * prepared layout (oproj.prepared page: the prepared object is the one that
 * binds the look-ahead, PreparedOproj.bind_ahead). Wp and Wp_bytes as for
 * attnres_oproj_packed_run; next_norm, next_query, next_eps, mixture,
 * ld_mixture and scal as for attnres_oproj_ahead_run. The statistics equal
 * attnres_oproj_ahead_run's bit for bit (they do not involve W); the other
 * outputs relate to attnres_oproj_ahead_run's as attnres_oproj_packed_run's
 * relate to attnres_oproj_run's.
 * Errors: those of attnres_oproj_packed_run and attnres_oproj_ahead_run.
 */
int attnres_oproj_packed_ahead_run(const void* x, int64_t ldx, const void* Wp, size_t Wp_bytes,
                                   int K, void* prefix, int64_t ld_prefix, void* blocks,
                                   int64_t blk_stride_t, int64_t blk_stride_b, int cap,
                                   const void* norm, const void* query, const void* out_norm,
                                   void* out, int64_t ld_out, void* aux, int64_t ld_aux, float eps,
                                   float out_eps, int M, int H, int nb, int write, int has_delta,
                                   int final_boundary, const void* next_norm,
                                   const void* next_query, float next_eps, float* mixture,
                                   int64_t ld_mixture, float* scal, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * attnres_post_run - attnres_run on carried saved-block statistics instead of
 * the saved blocks (ClusterAttnRes.post on the state pre leaves; the state
 * attnres_oproj_ahead_run stores). For every token t < T, with new and l_n as
 * for attnres_run and (m, S) = scal[t]:
 *   nb == 0 : h = new (mixture and scal are not read and may be NULL)
 *   nb >  0 : top = max(m, l_n), alpha = exp(m - top), e_n = exp(l_n - top),
 *             D = alpha S + e_n, h = (alpha mixture[t] + e_n new) / D,
 *             rounded to bf16 when final_boundary != 0
 *   out[t] = bf16(h * r(sum h^2, out_eps) * out_norm); the state writes of
 *   attnres_run (prefix, aux, blocks[t, write]).
 * Given the statistics attnres_run would form from the same blocks, norm,
 * query and eps, the outputs equal attnres_run's bit for bit. The saved
 * blocks are not read: blocks is written (slot write) only and may be NULL
 * when write == -1. nb (0..8) is the number of blocks the statistics cover.
 *   mixture [T, H] FP32, row stride ld_mixture >= H, a multiple of 8, 16-byte
 *   aligned; scal [T, 2] FP32, 8-byte aligned (both read).
 * Other arguments and errors as for attnres_run (nb need not be <= cap).
 */
int attnres_post_run(const void* delta, int64_t ld_delta, void* prefix, int64_t ld_prefix,
                     void* blocks, int64_t blk_stride_t, int64_t blk_stride_b, int cap,
                     const void* norm, const void* query, const void* out_norm, void* out,
                     int64_t ld_out, void* aux, int64_t ld_aux, const float* mixture,
                     int64_t ld_mixture, const float* scal, float eps, float out_eps, int T, int H,
                     int nb, int write, int has_delta, int final_boundary, void* stream);

/* attnres_strerror - a static, human-readable description of a return code. */
const char* attnres_strerror(int code);

/*
 * attnres_stream_read - a measurement helper, not a step of the method: it
 * reads `bytes` bytes at src exactly once with 16-byte non-temporal loads
 * spread over the whole device, the access pattern of a plain HBM stream,
 * so that the streaming-read bandwidth this device reaches can be set beside
 * the roofline figures of the kernels above. Each of its
 * ATTNRES_STREAM_READ_SINK_WORDS workgroups stores the XOR of the 32-bit words
 * it read to sink[workgroup] (so no load can be dropped); the XOR of all sink
 * words is the XOR of every word of src.
 *   src: device memory, 16-byte aligned, NULL only when bytes == 0;
 *   bytes: a multiple of 16.
 *   sink: device memory for ATTNRES_STREAM_READ_SINK_WORDS 32-bit words,
 *   4-byte aligned; every word is written.
 * Errors: ATTNRES_EINVAL (NULL sink or src), ATTNRES_EALIGN (src or bytes not
 * a multiple of 16, sink not 4-byte aligned), ATTNRES_EHIP.
 */
#define ATTNRES_STREAM_READ_SINK_WORDS 65536
int attnres_stream_read(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
