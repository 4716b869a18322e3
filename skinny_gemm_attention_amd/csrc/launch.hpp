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

// Counters of the fused kernel's single cross-workgroup hand-off. Zero between
// calls: the last consumer of a call resets them.
struct FusedSync {
  unsigned arrive;  // GEMM workgroups whose new-prefix columns are stored
  unsigned done;    // owner workgroups past the wait
};

struct FusedParams {
  AttnParams a;  // a.delta unused; a.T = M
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* W;
  int64_t ldw;
  int K;
  FusedSync* sync;
};

hipError_t launch_wsgemm(const GemmParams& p, hipStream_t stream);
hipError_t launch_attnres(const AttnParams& p, hipStream_t stream);
hipError_t launch_fused(const FusedParams& p, hipStream_t stream);

}  // namespace attnres
