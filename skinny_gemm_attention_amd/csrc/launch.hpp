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
// [M][H/2] 32-bit words (a bf16 pair each). Every mailbox word holds the
// sentinel between calls; a call's GEMM workgroups overwrite it with the new
// prefix and the owning workgroup re-arms it after reading.
constexpr unsigned kMailboxSentinel = 0x80000000u;  // bf16 pair (+0.0, -0.0)
constexpr size_t kWorkspaceHeader = 256;

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
  unsigned* mailbox;  // [M][H / 2]
};

hipError_t launch_wsgemm(const GemmParams& p, hipStream_t stream);
hipError_t launch_attnres(const AttnParams& p, hipStream_t stream);
hipError_t launch_fused(const FusedParams& p, hipStream_t stream);
hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t stream);

}  // namespace attnres
