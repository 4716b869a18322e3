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
  // MoE-front epilogue (moe != 0): y rows are out rows of width ldy; output
  // row c < valid goes as an FP32 word to bf16 column router_base + 2 (slot + c),
  // c >= split as bf16 to column base + c - split, the rows between nowhere
  int moe, router_base, slot, base, valid, split;
};

// Workspace of the fused kernel: a small header, then the new-prefix mailbox
// [M][H/2] 32-bit words (a bf16 pair each), then (beyond 32 tokens) the
// split-K hand-off: per 64-row group, the FP32 partial products of the
// workgroup that streams the even 4 KB blocks of K, one 16-byte quad per MFMA
// output quad. Every word after the header
// holds the sentinel between calls; a producer overwrites it and the consumer
// re-arms it after reading. 0x80000000 is the bf16 pair (+0.0, -0.0), which a
// new-prefix pair never holds, and the FP32 -0.0, which a stored partial
// never holds (producers store +0.0 for a zero).
constexpr unsigned kMailboxSentinel = 0x80000000u;
constexpr size_t kWorkspaceHeader = 256;

// Split-K hand-off bytes for M tokens and H rows (0 when no split is used).
constexpr size_t split_partial_bytes(int M, int H) {
  if (M <= 32) return 0;
  const size_t groups = (size_t)(H + 63) / 64;
  const size_t quads = 4 * (size_t)((M + 15) / 16) * 64;  // four row tiles x token tiles
  return groups * quads * 16;
}

// Polling of sentinel-armed words: one 16-byte device-scope (sc1) buffer load
// per pending piece per round, all issued back to back; a piece that has
// already arrived gets an offset past the end of the buffer, which the
// hardware answers with zeros and no memory access. Every wait is bounded by
// kSpinLimit rounds (about a second); a workgroup that gives up flags the
// workspace and finishes.
constexpr int kSpinLimit = 1 << 20;
constexpr int kCacheSC1 = 16;  // buffer-load cache policy: device scope

// Hand-off bytes of wsgemm_run_ws for M tokens and N rows: up to three parts
// per 64-row group (four-way split), one 16-byte quad per MFMA output quad.
inline size_t wsgemm_split_partial_bytes(int M, int N) {
  if (M <= 32) return 0;
  const size_t groups = (size_t)(N + 63) / 64;
  const size_t quads = 4 * (size_t)((M + 15) / 16) * 64;
  return 3 * groups * quads * 16;
}

struct FusedWorkspace {
  // nonzero after a wait gave up (that call's results are invalid); every
  // later call on the workspace then writes nothing until it is re-armed
  unsigned error;
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
  int wrows;           // 0: W row-major (row stride ldw); else W prepared (pack_kernel) with wrows rows
  AheadParams ah;      // ah.mix == nullptr: no look-ahead statistics
};

// The prepared (tile-major) layout of a W [N, K] bf16 (pack_kernel):
// P = 4 ceil(K / 512) planes of 128 k-values; plane j holds every row's
// k-values [128 j, 128 j + 128) as one 256-byte segment, rows in order, and
// within the segment of row n the 16-byte piece p (k-values 8p .. 8p + 7) sits
// at position p ^ (n & 15); k-values at or past K are zero.
inline size_t packed_planes(int K) { return 4 * (((size_t)K + 511) / 512); }
inline size_t packed_bytes(int N, int K) { return packed_planes(K) * (size_t)N * 256; }

int compute_units();
hipError_t launch_wsgemm(const GemmParams& p, hipStream_t stream);
// Split K over up to four workgroups per 64-row group beyond 32 tokens (when
// the parts fit `compute_units`), else launch_wsgemm. The workspace holds the
// 256-byte header, then the hand-off of wsgemm_split_partial_bytes(M, N).
hipError_t launch_wsgemm_ws(const GemmParams& p, void* workspace, int compute_units,
                            hipStream_t stream);
// Whether launch_wsgemm_ws splits K for this shape (beyond 64 tokens it must).
bool wsgemm_ws_splits(int M, int N, int K, int compute_units);
hipError_t launch_attnres(const AttnParams& p, hipStream_t stream);
hipError_t launch_fused(const FusedParams& p, hipStream_t stream);
hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t stream);
hipError_t launch_pack_weights(const uint16_t* W, int64_t ldw, int N, int K, uint16_t* Wp,
                               hipStream_t stream);

}  // namespace attnres
