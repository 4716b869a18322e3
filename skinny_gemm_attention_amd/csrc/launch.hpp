// Kernel launchers shared by the C-ABI layer (arguments already validated).
#pragma once

#include "token.hpp"

namespace attnres {

struct GemmParams {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* W;
  int64_t ldw;
  uint16_t* y;
  int64_t ldy;
  int M, N, K;
};

// Workspace of the fused kernel: a small header, then the new-prefix mailbox
// [M][H/2] 32-bit words (a bf16 pair each), then (beyond 32 tokens) the
// split-K hand-off: per 64-row group, the first K half's FP32 partial
// products, one 16-byte quad per MFMA output quad. Every word after the header
// holds the sentinel between calls; a producer overwrites it and the consumer
// re-arms it after reading. 0x80000000 is the bf16 pair (+0.0, -0.0), which a
// new-prefix pair never holds, and the FP32 -0.0, which a stored partial
// never holds (producers store +0.0 for a zero).
constexpr unsigned kMailboxSentinel = 0x80000000u;
constexpr size_t kWorkspaceHeader = 256;

// Split-K hand-off bytes for M tokens and H rows (0 when no split is used).
inline size_t split_partial_bytes(int M, int H) {
  if (M <= 32) return 0;
  const size_t groups = (size_t)(H + 63) / 64;
  const size_t quads = 4 * (size_t)((M + 15) / 16) * 64;  // four row tiles x token tiles
  return groups * quads * 16;
}

struct FusedWorkspace {
  unsigned error;  // nonzero after an owner gave up waiting (results invalid)
};

struct FusedParams {
  AttnParams a;  // a.delta unused; a.T = M
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* W;
  int64_t ldw;
  int K;
  FusedWorkspace* ws;
  unsigned* mailbox;   // [M][H / 2]
  unsigned* partials;  // split-K hand-off (see above)
  int ng;              // split-K row groups (0: no split)
  AheadParams ah;      // ah.mix == nullptr: no look-ahead statistics
};

hipError_t launch_wsgemm(const GemmParams& p, hipStream_t stream);
hipError_t launch_attnres(const AttnParams& p, hipStream_t stream);
hipError_t launch_fused(const FusedParams& p, hipStream_t stream);
hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t stream);

}  // namespace attnres
