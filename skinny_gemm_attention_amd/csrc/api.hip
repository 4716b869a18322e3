// C ABI of the decode-step hot path (declared in include/attnres.h).
//
// Every argument is checked here, on the host, before any HIP call: an invalid
// call returns a negative code and enqueues nothing.
#include "../../include/attnres.h"
#include "launch.hpp"

#include <mutex>

namespace attnres {
// stream_read.hip: reads `bytes` (a multiple of 16) at src once; workgroup
// g < grid stores the XOR of the words it read to sink[g].
hipError_t launch_stream_read(const void* src, size_t bytes, unsigned* sink, int grid,
                              hipStream_t stream);
}  // namespace attnres

namespace {

using attnres::AttnParams;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride8(int64_t s) { return s >= 0 && (s & 7) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? ATTNRES_OK : ATTNRES_EHIP; }

// Checks shared by attnres_run and attnres_oproj_run (T tokens).
int check_attnres(const void* prefix, int64_t ld_prefix, const void* blocks, int64_t bst_t,
                  int64_t bst_b, int cap, const void* norm, const void* query,
                  const void* out_norm, const void* out, int64_t ld_out, const void* aux,
                  int64_t ld_aux, float eps, float out_eps, int T, int H, int nb, int write,
                  int has_delta, int final_boundary) {
  if (T < 0 || H < 0 || cap < 0) return ATTNRES_EINVAL;
  if ((has_delta != 0 && has_delta != 1) || (final_boundary != 0 && final_boundary != 1))
    return ATTNRES_EINVAL;
  if (!prefix || !norm || !query || !out_norm || !out) return ATTNRES_EINVAL;
  if (!(eps >= 0.0f) || !(out_eps >= 0.0f) || eps > 1e30f || out_eps > 1e30f) return ATTNRES_EINVAL;
  if (H < 8 || H > ATTNRES_MAX_H || (H & 7)) return ATTNRES_EUNSUPPORTED;
  if (nb < 0 || nb > ATTNRES_MAX_BLOCKS || nb > cap) return ATTNRES_ERANGE;
  if (write < -1 || write >= cap) return ATTNRES_ERANGE;
  const bool uses_blocks = nb > 0 || write >= 0;
  if (uses_blocks && !blocks) return ATTNRES_EINVAL;
  if (ld_prefix < H || ld_out < H || (aux && ld_aux < H)) return ATTNRES_EINVAL;
  if (!aligned16(prefix) || !aligned16(norm) || !aligned16(query) || !aligned16(out_norm) ||
      !aligned16(out) || (aux && !aligned16(aux)) || (uses_blocks && !aligned16(blocks)))
    return ATTNRES_EALIGN;
  if (!stride8(ld_prefix) || !stride8(ld_out) || (aux && !stride8(ld_aux))) return ATTNRES_EALIGN;
  if (uses_blocks) {
    if (bst_t < H || bst_b < H) return ATTNRES_EINVAL;
    if (!stride8(bst_t) || !stride8(bst_b)) return ATTNRES_EALIGN;
    const bool token_major = bst_t >= (int64_t)cap * bst_b;
    const bool slot_major = bst_b >= (int64_t)T * bst_t;
    if (!token_major && !slot_major) return ATTNRES_EINVAL;  // rows would overlap
  }
  return ATTNRES_OK;
}

AttnParams make_params(const void* delta, int64_t ld_delta, void* prefix, int64_t ld_prefix,
                       void* blocks, int64_t bst_t, int64_t bst_b, const void* norm,
                       const void* query, const void* out_norm, void* out, int64_t ld_out,
                       void* aux, int64_t ld_aux, float eps, float out_eps, int T, int H, int nb,
                       int write, int has_delta, int final_boundary) {
  AttnParams p;
  p.delta = static_cast<const uint16_t*>(delta);
  p.ld_delta = ld_delta;
  p.prefix = static_cast<uint16_t*>(prefix);
  p.ld_prefix = ld_prefix;
  p.blocks = static_cast<uint16_t*>(blocks);
  p.bst_t = bst_t;
  p.bst_b = bst_b;
  p.norm = static_cast<const uint16_t*>(norm);
  p.query = static_cast<const uint16_t*>(query);
  p.out_norm = static_cast<const uint16_t*>(out_norm);
  p.out = static_cast<uint16_t*>(out);
  p.ld_out = ld_out;
  p.aux = static_cast<uint16_t*>(aux);
  p.ld_aux = ld_aux;
  p.eps = eps;
  p.out_eps = out_eps;
  p.inv_h = 1.0f / (float)H;
  p.T = T;
  p.H = H;
  p.nb = nb;
  p.write = write;
  p.has_delta = has_delta;
  p.final_b = final_boundary;
  p.smix = nullptr;
  p.ld_smix = 0;
  p.sscal = nullptr;
  return p;
}

// Checks of carried saved-block statistics: mixture [T, H] FP32 with row
// stride ld_mix, scal [T, 2] FP32. Unused (and may be NULL) when nb == 0.
int check_stats(const void* mixture, int64_t ld_mix, const void* scal, int H, int nb) {
  if (nb == 0) return ATTNRES_OK;
  if (!mixture || !scal) return ATTNRES_EINVAL;
  if (ld_mix < H) return ATTNRES_EINVAL;
  if (!aligned16(mixture) || (reinterpret_cast<uintptr_t>(scal) & 7u)) return ATTNRES_EALIGN;
  if (!stride8(ld_mix)) return ATTNRES_EALIGN;
  return ATTNRES_OK;
}

// Header, one bf16 mailbox row per token, and (beyond 32 tokens) the split-K
// hand-off.
size_t mailbox_bytes(int M, int H) {
  const size_t mailbox = (size_t)M * (size_t)H * 2;
  return (mailbox + 255) & ~(size_t)255;
}
size_t workspace_bytes_for(int M, int H) {
  if (M < 0 || H < 0) return 0;
  return attnres::kWorkspaceHeader + mailbox_bytes(M, H) + attnres::split_partial_bytes(M, H);
}

}  // namespace

extern "C" {

int attnres_run(const void* delta, int64_t ld_delta, void* prefix, int64_t ld_prefix,
                void* blocks, int64_t blk_stride_t, int64_t blk_stride_b, int cap,
                const void* norm, const void* query, const void* out_norm, void* out,
                int64_t ld_out, void* aux, int64_t ld_aux, float eps, float out_eps, int T,
                int H, int nb, int write, int has_delta, int final_boundary, void* stream) {
  if (T < 0) return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // nothing to read or write
  int rc = check_attnres(prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b, cap, norm, query,
                         out_norm, out, ld_out, aux, ld_aux, eps, out_eps, T, H, nb, write,
                         has_delta, final_boundary);
  if (rc) return rc;
  if (!delta) return ATTNRES_EINVAL;
  if (ld_delta < H) return ATTNRES_EINVAL;
  if (!aligned16(delta)) return ATTNRES_EALIGN;
  if (!stride8(ld_delta)) return ATTNRES_EALIGN;
  AttnParams p = make_params(delta, ld_delta, prefix, ld_prefix, blocks, blk_stride_t,
                             blk_stride_b, norm, query, out_norm, out, ld_out, aux, ld_aux, eps,
                             out_eps, T, H, nb, write, has_delta, final_boundary);
  return from_hip(attnres::launch_attnres(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks of wsgemm_run's arguments (M > 0); fills p. y rows hold N elements
// unless `any_width` (the MoE-front epilogue checks its own columns).
int check_gemm(const void* x, int64_t ldx, const void* W, int64_t ldw, void* y, int64_t ldy,
               int M, int N, int K, attnres::GemmParams& p, bool any_width = false,
               int max_m = ATTNRES_MAX_M) {
  if (!y || (K > 0 && (!x || !W))) return ATTNRES_EINVAL;  // x, W unread when K == 0
  if (M > max_m) return ATTNRES_ERANGE;
  if (N < 8 || (N & 7) || (K & 7)) return ATTNRES_EUNSUPPORTED;
  if ((!any_width && ldy < N) || ldy < 0 || (K > 0 && (ldx < K || ldw < K))) return ATTNRES_EINVAL;
  if (!aligned16(y) || (K > 0 && (!aligned16(x) || !aligned16(W)))) return ATTNRES_EALIGN;
  if (!stride8(ldy) || (K > 0 && (!stride8(ldx) || !stride8(ldw)))) return ATTNRES_EALIGN;
  p.x = static_cast<const uint16_t*>(x);
  p.ldx = ldx;
  p.W = static_cast<const uint16_t*>(W);
  p.ldw = ldw;
  p.y = static_cast<uint16_t*>(y);
  p.ldy = ldy;
  p.M = M;
  p.N = N;
  p.K = K;
  p.moe = p.router_base = p.slot = p.base = p.valid = p.split = 0;
  return ATTNRES_OK;
}

}  // namespace

extern "C" {

size_t wsgemm_workspace_size(int M, int N) {
  if (M < 0 || N < 0) return 0;
  return attnres::kWorkspaceHeader + attnres::wsgemm_split_partial_bytes(M, N);
}

int wsgemm_run_ws(const void* x, int64_t ldx, const void* W, int64_t ldw, void* y, int64_t ldy,
                  int M, int N, int K, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return ATTNRES_EINVAL;
  if (M == 0) return ATTNRES_OK;  // nothing to read or write
  attnres::GemmParams p;
  int rc = check_gemm(x, ldx, W, ldw, y, ldy, M, N, K, p, false, ATTNRES_MAX_M_WS);
  if (rc) return rc;
  if (M > ATTNRES_MAX_M && !attnres::wsgemm_ws_splits(M, N, K, attnres::compute_units()))
    return ATTNRES_EUNSUPPORTED;  // beyond 64 tokens only the split kernel serves
  if (!workspace || workspace_bytes < wsgemm_workspace_size(M, N) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return ATTNRES_EWORKSPACE;
  return from_hip(attnres::launch_wsgemm_ws(p, workspace, attnres::compute_units(),
                                            static_cast<hipStream_t>(stream)));
}

int wsgemm_moe_front_run(const void* x, int64_t ldx, const void* W, int64_t ldw, void* out,
                         int64_t ld_out, int M, int N, int K, int router_base, int slot, int base,
                         int valid, int split, void* stream) {
  if (M < 0 || N < 0 || K < 0) return ATTNRES_EINVAL;
  if (M == 0) return ATTNRES_OK;  // nothing to read or write
  attnres::GemmParams p;
  int rc = check_gemm(x, ldx, W, ldw, out, ld_out, M, N, K, p, true);
  if (rc) return rc;
  if (router_base < 0 || slot < 0 || base < 0 || valid < 0 || split < valid || split > N)
    return ATTNRES_ERANGE;
  if ((valid & 7) || (split & 7) || (router_base & 1) || (base & 1)) return ATTNRES_EALIGN;
  if (valid > 0 && (int64_t)router_base + 2 * ((int64_t)slot + valid) > ld_out) return ATTNRES_ERANGE;
  if (split < N && (int64_t)base + (N - split) > ld_out) return ATTNRES_ERANGE;
  if (valid > 0 && split < N) {  // the two shards must not overlap
    const int64_t r0 = (int64_t)router_base + 2 * (int64_t)slot, r1 = r0 + 2 * (int64_t)valid;
    const int64_t l0 = base, l1 = (int64_t)base + (N - split);
    if (r0 < l1 && l0 < r1) return ATTNRES_ERANGE;
  }
  p.moe = 1;
  p.router_base = router_base;
  p.slot = slot;
  p.base = base;
  p.valid = valid;
  p.split = split;
  return from_hip(attnres::launch_wsgemm(p, static_cast<hipStream_t>(stream)));
}

int wsgemm_run(const void* x, int64_t ldx, const void* W, int64_t ldw, void* y, int64_t ldy,
               int M, int N, int K, void* stream) {
  if (M < 0 || N < 0 || K < 0) return ATTNRES_EINVAL;
  if (M == 0) return ATTNRES_OK;  // nothing to read or write
  attnres::GemmParams p;
  int rc = check_gemm(x, ldx, W, ldw, y, ldy, M, N, K, p);
  if (rc) return rc;
  return from_hip(attnres::launch_wsgemm(p, static_cast<hipStream_t>(stream)));
}

size_t attnres_oproj_workspace_size(int M, int H, int nb) {
  (void)nb;
  return workspace_bytes_for(M, H);
}

int attnres_oproj_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < attnres::kWorkspaceHeader) return ATTNRES_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) || (workspace_bytes & 3u))
    return ATTNRES_EWORKSPACE;
  return from_hip(attnres::launch_workspace_init(workspace, workspace_bytes,
                                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// ---- the library's own workspace (attnres_oproj_run_noalloc) -----------------
//
// For callers that cannot allocate, the workspace of attnres_oproj_run lives
// in a file-scope device array, one copy per device, held until the process
// ends: the largest workspace the fused call can need (64 tokens, H = 8192;
// 3,145,984 bytes). On the host, `scratch` is only a stand-in for the device
// copies: its address on a device comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is ever
// handed to a kernel or a copy.
constexpr size_t kStaticWorkspaceBytes = attnres::kWorkspaceHeader +
                                         (size_t)ATTNRES_MAX_M * ATTNRES_MAX_H * 2 +
                                         attnres::split_partial_bytes(ATTNRES_MAX_M, ATTNRES_MAX_H);
static_assert(kStaticWorkspaceBytes == ATTNRES_NOALLOC_WORKSPACE_BYTES, "header figure");
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
struct StaticWorkspace {
  void* ptr = nullptr;  // device address of `scratch` on this device
  bool armed = false;   // an arming kernel has run (not merely been captured) on it
};
std::mutex g_static_mu;
StaticWorkspace g_static[kMaxDevices];

// The device `stream` belongs to, which must be the current device.
int stream_device(hipStream_t stream, int* dev) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return ATTNRES_EHIP;
  if (stream) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return ATTNRES_EHIP;
    if ((int)sd != cur) return ATTNRES_EINVAL;
  }
  if (cur < 0 || cur >= kMaxDevices) return ATTNRES_EINVAL;
  *dev = cur;
  return ATTNRES_OK;
}

// The current device's copy of `scratch`, armed before its first use: the
// arming kernel is enqueued on `stream` ahead of the call that needs it. When
// `stream` is being captured, the arming kernel goes into the graph (every
// replay re-arms the array, which is harmless) and the device still counts
// as unarmed, so the next call outside a capture arms it again.
int static_workspace(hipStream_t stream, void** ws) {
  int dev = 0;
  int rc = stream_device(stream, &dev);
  if (rc) return rc;
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticWorkspace& st = g_static[dev];
  if (!st.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTNRES_EHIP;
    st.ptr = p;
  }
  if (!st.armed) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return ATTNRES_EHIP;
    if (attnres::launch_workspace_init(st.ptr, kStaticWorkspaceBytes, stream) != hipSuccess)
      return ATTNRES_EHIP;
    if (cs == hipStreamCaptureStatusNone) st.armed = true;
  }
  *ws = st.ptr;
  return ATTNRES_OK;
}

// The current device's copy of `scratch` if a call has used it, else nullptr.
int static_workspace_if_used(hipStream_t stream, void** ws) {
  int dev = 0;
  int rc = stream_device(stream, &dev);
  if (rc) return rc;
  std::lock_guard<std::mutex> lock(g_static_mu);
  *ws = g_static[dev].ptr;
  return ATTNRES_OK;
}

// Checks of the look-ahead arguments (attnres_oproj_ahead_run and its
// prepared-W form); fills `ah` when they pass.
int ahead_params(const void* next_norm, const void* next_query, float next_eps, float* mixture,
                 int64_t ld_mixture, float* scal, int H, attnres::AheadParams* ah) {
  if (!next_norm || !next_query || !mixture || !scal) return ATTNRES_EINVAL;
  if (!(next_eps >= 0.0f) || next_eps > 1e30f) return ATTNRES_EINVAL;
  if (H >= 8 && H <= ATTNRES_MAX_H && !(H & 7)) {  // other H: rejected by the fused checks
    if (ld_mixture < H) return ATTNRES_EINVAL;
  }
  if (!aligned16(next_norm) || !aligned16(next_query) || !aligned16(mixture) ||
      (reinterpret_cast<uintptr_t>(scal) & 7u))
    return ATTNRES_EALIGN;
  if (!stride8(ld_mixture)) return ATTNRES_EALIGN;
  *ah = attnres::AheadParams{static_cast<const uint16_t*>(next_norm),
                             static_cast<const uint16_t*>(next_query), next_eps, mixture,
                             ld_mixture, scal};
  return ATTNRES_OK;
}

// Checks and launch of the fused call; with `library_ws` the workspace is the
// library's own (attnres_oproj_run_noalloc) and `workspace` is ignored.
int oproj_common(const void* x, int64_t ldx, const void* W, int64_t ldw, int K, void* prefix,
                 int64_t ld_prefix, void* blocks, int64_t blk_stride_t, int64_t blk_stride_b,
                 int cap, const void* norm, const void* query, const void* out_norm, void* out,
                 int64_t ld_out, void* aux, int64_t ld_aux, float eps, float out_eps, int M, int H,
                 int nb, int write, int has_delta, int final_boundary, void* workspace,
                 size_t workspace_bytes, const attnres::AheadParams& ah, void* stream,
                 bool library_ws = false, bool packed_w = false, size_t w_bytes = 0) {
  int rc = check_attnres(prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b, cap, norm, query,
                         out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H, nb, write,
                         has_delta, final_boundary);
  if (rc) return rc;
  if (K < 0 || (K > 0 && (!x || !W))) return ATTNRES_EINVAL;  // x, W unread when K == 0
  if (M < 1 || M > ATTNRES_MAX_M) return ATTNRES_ERANGE;
  if (K & 7) return ATTNRES_EUNSUPPORTED;
  if (K > 0 && (ldx < K || (!packed_w && ldw < K))) return ATTNRES_EINVAL;
  if (K > 0 && packed_w && w_bytes < attnres::packed_bytes(H, K)) return ATTNRES_EINVAL;
  if (K > 0 && packed_w && attnres::packed_bytes(H, K) >= ((size_t)1 << 32))
    return ATTNRES_EUNSUPPORTED;  // prepared W is addressed with 32-bit offsets
  if (K > 0 && (!aligned16(x) || !aligned16(W))) return ATTNRES_EALIGN;
  if (K > 0 && (!stride8(ldx) || (!packed_w && !stride8(ldw)))) return ATTNRES_EALIGN;
  if (library_ws) {
    // never reached within the limits above: the array covers 64 tokens of
    // the widest rows
    if (workspace_bytes_for(M, H) > kStaticWorkspaceBytes) return ATTNRES_EWORKSPACE;
    rc = static_workspace(static_cast<hipStream_t>(stream), &workspace);
    if (rc) return rc;
    workspace_bytes = kStaticWorkspaceBytes;
  }
  if (!workspace || workspace_bytes < workspace_bytes_for(M, H) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return ATTNRES_EWORKSPACE;
  attnres::FusedParams p;
  p.a = make_params(nullptr, 0, prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b, norm, query,
                    out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H, nb, write, has_delta,
                    final_boundary);
  p.x = static_cast<const uint16_t*>(x);
  p.ldx = ldx;
  p.W = static_cast<const uint16_t*>(W);
  p.ldw = ldw;
  p.K = K;
  p.ws = static_cast<attnres::FusedWorkspace*>(workspace);
  p.mailbox = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + attnres::kWorkspaceHeader);
  p.partials = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) +
                                           attnres::kWorkspaceHeader + mailbox_bytes(M, H));
  p.ng = 0;
  p.wrows = packed_w ? H : 0;
  p.ah = ah;
  return from_hip(attnres::launch_fused(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int attnres_oproj_run(const void* x, int64_t ldx, const void* W, int64_t ldw, int K, void* prefix,
                      int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                      int64_t blk_stride_b, int cap, const void* norm, const void* query,
                      const void* out_norm, void* out, int64_t ld_out, void* aux, int64_t ld_aux,
                      float eps, float out_eps, int M, int H, int nb, int write, int has_delta,
                      int final_boundary, void* workspace, size_t workspace_bytes,
                      void* stream) {
  attnres::AheadParams ah = {nullptr, nullptr, 0.0f, nullptr, 0, nullptr};
  return oproj_common(x, ldx, W, ldw, K, prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b,
                      cap, norm, query, out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H,
                      nb, write, has_delta, final_boundary, workspace, workspace_bytes, ah,
                      stream);
}

size_t attnres_packed_weights_size(int N, int K) {
  if (N < 0 || K < 0) return 0;
  return attnres::packed_bytes(N, K);
}

int attnres_pack_weights(const void* W, int64_t ldw, int N, int K, void* Wp, size_t Wp_bytes,
                         void* stream) {
  if (N < 0 || K < 0) return ATTNRES_EINVAL;
  if (N == 0 || K == 0) return ATTNRES_OK;  // nothing to read or write
  if (!W || !Wp || ldw < K) return ATTNRES_EINVAL;
  if ((K & 7) || N > (1 << 24)) return ATTNRES_EUNSUPPORTED;
  if (!aligned16(W) || !aligned16(Wp) || !stride8(ldw)) return ATTNRES_EALIGN;
  if (Wp_bytes < attnres::packed_bytes(N, K)) return ATTNRES_EINVAL;
  return from_hip(attnres::launch_pack_weights(static_cast<const uint16_t*>(W), ldw, N, K,
                                               static_cast<uint16_t*>(Wp),
                                               static_cast<hipStream_t>(stream)));
}

int attnres_oproj_packed_run(const void* x, int64_t ldx, const void* Wp, size_t Wp_bytes, int K,
                             void* prefix, int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                             int64_t blk_stride_b, int cap, const void* norm, const void* query,
                             const void* out_norm, void* out, int64_t ld_out, void* aux,
                             int64_t ld_aux, float eps, float out_eps, int M, int H, int nb,
                             int write, int has_delta, int final_boundary, void* workspace,
                             size_t workspace_bytes, void* stream) {
  attnres::AheadParams ah = {nullptr, nullptr, 0.0f, nullptr, 0, nullptr};
  return oproj_common(x, ldx, Wp, 0, K, prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b,
                      cap, norm, query, out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H,
                      nb, write, has_delta, final_boundary, workspace, workspace_bytes, ah, stream,
                      false, true, Wp_bytes);
}

int attnres_oproj_run_noalloc(const void* x, int64_t ldx, const void* W, int64_t ldw, int K,
                              void* prefix, int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                              int64_t blk_stride_b, int cap, const void* norm, const void* query,
                              const void* out_norm, void* out, int64_t ld_out, void* aux,
                              int64_t ld_aux, float eps, float out_eps, int M, int H, int nb,
                              int write, int has_delta, int final_boundary, void* stream) {
  attnres::AheadParams ah = {nullptr, nullptr, 0.0f, nullptr, 0, nullptr};
  return oproj_common(x, ldx, W, ldw, K, prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b,
                      cap, norm, query, out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H,
                      nb, write, has_delta, final_boundary, nullptr, 0, ah, stream, true);
}

int attnres_oproj_ahead_run(const void* x, int64_t ldx, const void* W, int64_t ldw, int K,
                            void* prefix, int64_t ld_prefix, void* blocks, int64_t blk_stride_t,
                            int64_t blk_stride_b, int cap, const void* norm, const void* query,
                            const void* out_norm, void* out, int64_t ld_out, void* aux,
                            int64_t ld_aux, float eps, float out_eps, int M, int H, int nb,
                            int write, int has_delta, int final_boundary,
                            const void* next_norm, const void* next_query, float next_eps,
                            float* mixture, int64_t ld_mixture, float* scal, void* workspace,
                            size_t workspace_bytes, void* stream) {
  attnres::AheadParams ah;
  const int rc = ahead_params(next_norm, next_query, next_eps, mixture, ld_mixture, scal, H, &ah);
  if (rc) return rc;
  return oproj_common(x, ldx, W, ldw, K, prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b,
                      cap, norm, query, out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H,
                      nb, write, has_delta, final_boundary, workspace, workspace_bytes, ah,
                      stream);
}

int attnres_oproj_packed_ahead_run(const void* x, int64_t ldx, const void* Wp, size_t Wp_bytes,
                                   int K, void* prefix, int64_t ld_prefix, void* blocks,
                                   int64_t blk_stride_t, int64_t blk_stride_b, int cap,
                                   const void* norm, const void* query, const void* out_norm,
                                   void* out, int64_t ld_out, void* aux, int64_t ld_aux, float eps,
                                   float out_eps, int M, int H, int nb, int write, int has_delta,
                                   int final_boundary, const void* next_norm,
                                   const void* next_query, float next_eps, float* mixture,
                                   int64_t ld_mixture, float* scal, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  attnres::AheadParams ah;
  const int rc = ahead_params(next_norm, next_query, next_eps, mixture, ld_mixture, scal, H, &ah);
  if (rc) return rc;
  return oproj_common(x, ldx, Wp, 0, K, prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b,
                      cap, norm, query, out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H,
                      nb, write, has_delta, final_boundary, workspace, workspace_bytes, ah, stream,
                      false, true, Wp_bytes);
}

int attnres_post_run(const void* delta, int64_t ld_delta, void* prefix, int64_t ld_prefix,
                     void* blocks, int64_t blk_stride_t, int64_t blk_stride_b, int cap,
                     const void* norm, const void* query, const void* out_norm, void* out,
                     int64_t ld_out, void* aux, int64_t ld_aux, const float* mixture,
                     int64_t ld_mixture, const float* scal, float eps, float out_eps, int T, int H,
                     int nb, int write, int has_delta, int final_boundary, void* stream) {
  if (T < 0) return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // nothing to read or write
  // the blocks are only written here: validate them as for a call that scores none
  int rc = check_attnres(prefix, ld_prefix, blocks, blk_stride_t, blk_stride_b, cap, norm, query,
                         out_norm, out, ld_out, aux, ld_aux, eps, out_eps, T, H, 0, write,
                         has_delta, final_boundary);
  if (rc) return rc;
  if (nb < 0 || nb > ATTNRES_MAX_BLOCKS) return ATTNRES_ERANGE;
  rc = check_stats(mixture, ld_mixture, scal, H, nb);
  if (rc) return rc;
  if (!delta) return ATTNRES_EINVAL;
  if (ld_delta < H) return ATTNRES_EINVAL;
  if (!aligned16(delta)) return ATTNRES_EALIGN;
  if (!stride8(ld_delta)) return ATTNRES_EALIGN;
  AttnParams p = make_params(delta, ld_delta, prefix, ld_prefix, blocks, blk_stride_t,
                             blk_stride_b, norm, query, out_norm, out, ld_out, aux, ld_aux, eps,
                             out_eps, T, H, nb, write, has_delta, final_boundary);
  // nb == 0 reads no statistics: the plain kernel gives the same result
  if (nb > 0) {
    p.smix = mixture;
    p.ld_smix = ld_mixture;
    p.sscal = scal;
  }
  return from_hip(attnres::launch_attnres(p, static_cast<hipStream_t>(stream)));
}

int attnres_workspace_status(const void* workspace, size_t workspace_bytes, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!workspace && workspace_bytes == 0) {  // the library's own (attnres_oproj_run_noalloc)
    void* own = nullptr;
    const int rc = static_workspace_if_used(s, &own);
    if (rc) return rc;
    if (!own) return ATTNRES_OK;  // no call has used it on this device
    workspace = own;
    workspace_bytes = kStaticWorkspaceBytes;
  }
  if (!workspace || workspace_bytes < attnres::kWorkspaceHeader ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return ATTNRES_EWORKSPACE;
  unsigned word = 0;
  if (hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return ATTNRES_EHIP;
  return word == 0 ? ATTNRES_OK : ATTNRES_EWAIT;
}

int attnres_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!sink || (!src && bytes > 0)) return ATTNRES_EINVAL;
  if ((bytes & 15u) != 0 || (src && !aligned16(src)) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return ATTNRES_EALIGN;
  return from_hip(attnres::launch_stream_read(src, bytes, static_cast<unsigned*>(sink),
                                              ATTNRES_STREAM_READ_SINK_WORDS,
                                              static_cast<hipStream_t>(stream)));
}

const char* attnres_strerror(int code) {
  switch (code) {
    case ATTNRES_OK: return "success";
    case ATTNRES_EINVAL: return "invalid argument (null pointer, size or stride)";
    case ATTNRES_EALIGN: return "pointer not 16-byte aligned or stride not a multiple of 8 elements";
    case ATTNRES_ERANGE: return "nb, write, cap, M or T out of range";
    case ATTNRES_EUNSUPPORTED: return "shape not supported (H, N or K limits)";
    case ATTNRES_EWORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case ATTNRES_EHIP: return "HIP launch failed";
    case ATTNRES_EWAIT:
      return "a wait in an earlier call on this workspace gave up: that call's results are invalid "
             "and later calls write nothing until attnres_oproj_workspace_init re-arms it";
    default: return "unknown error code";
  }
}

}  // extern "C"
