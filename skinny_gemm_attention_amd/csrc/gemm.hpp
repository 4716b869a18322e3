// Weight-stationary skinny GEMM core on the MFMA units of gfx950.
//
// The operation is WsGemm's y[M, N] = x[M, K] W[N, K]^T (vLLM gemm.ws_gemm
// page, module summary) for M <= 64 tokens: BF16 operands, FP32 accumulation,
// K partial sums added in K order. The layout is ours:
//
//   * A workgroup owns R consecutive rows of W (R = 4..32, a multiple of 4: 256
//     workgroups of 28 rows for 7168 rows) and all K; its NW wavefronts split K
//     into NW consecutive ranges of 32-wide k-steps. Each x fragment a
//     wavefront loads serves all of the workgroup's rows.
//   * Per k-step a wavefront issues v_mfma_f32_16x16x32_bf16 with W as the A
//     operand (16 rows x 32 k) and x as the B operand (32 k x 16 tokens), one
//     MFMA per (16-row tile rt < RT, 16-token tile tt < TT). Lane l loads 16
//     contiguous bytes: W row (l % 16), x token (l % 16), k = 32 s + 8 (l / 16).
//     Rows past R, tokens past M and k past K load as zero.
//   * W is streamed once with non-temporal 16-byte loads, D k-steps per stage,
//     double-buffered so that the next stage's loads are in flight while the
//     current stage's MFMAs run. x (at most 1 MiB) stays in L2.
//   * The NW partial tiles are summed in LDS in wavefront order (= K order).
//
// The MFMA accumulator of lane l holds D[4 (l / 16) + r][l % 16], r < 4: rows
// n0 + 4 (l / 16) + r of token (l % 16) of the tile.
#pragma once

#include "common.hpp"

namespace attnres {

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int RT, int TT, int NW, int D>
struct GemmCore {
  static constexpr int NT = NW * 64;
  static constexpr int kQuads = RT * TT * 64;  // (tile, lane) pairs of one workgroup tile

  // Per-wavefront streaming state. start() computes the operand addresses and
  // issues the first stage of loads; finish() runs the pipelined K loop, so a
  // caller can put other work between the two while those loads are in flight.
  const uint16_t* wp[RT];
  const uint16_t* xp[TT];
  bool wv[RT], xv[TT];
  int s, s1, kq, K;
  u32x4 wa[D][RT], xa[D][TT], wb[D][RT], xb[D][TT];
  f32x4 acc[RT][TT];

  __device__ __forceinline__ void load(u32x4 (&wr)[D][RT], u32x4 (&xr)[D][TT], int st) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // this lane's 8 elements start at k; K % 8 == 0, so k < K implies k + 8 <= K
      const int k = (st + d) * 32 + kq * 8;
      const bool kv = (st + d < s1) && (k < K);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) wr[d][rt] = (kv && wv[rt]) ? ld16_stream(wp[rt] + k) : zero;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) xr[d][tt] = (kv && xv[tt]) ? ld16(xp[tt] + k) : zero;
    }
  }

  __device__ __forceinline__ void mma(const u32x4 (&wr)[D][RT], const u32x4 (&xr)[D][TT], int st) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (st + d < s1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = mfma_bf16(wr[d][rt], xr[d][tt], acc[rt][tt]);
      }
    }
  }

  // This wavefront's K range of the workgroup's [rows x M] tile.
  __device__ __forceinline__ void start(const uint16_t* __restrict__ x, int64_t ldx,
                                        const uint16_t* __restrict__ W, int64_t ldw, int M,
                                        int K_, int row0, int rows) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    kq = lane >> 4;
    K = K_;
    const int S = (K + 31) >> 5;
    s = (S * wave) / NW;
    s1 = (S * (wave + 1)) / NW;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + r16;
      wv[rt] = r < rows;
      wp[rt] = W + (size_t)(row0 + (wv[rt] ? r : 0)) * ldw;
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int m = tt * 16 + r16;
      xv[tt] = m < M;
      xp[tt] = x + (size_t)(xv[tt] ? m : 0) * ldx;
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (s < s1) load(wa, xa, s);
  }

  __device__ __forceinline__ void finish() {
    while (s < s1) {
      if (s + D < s1) load(wb, xb, s + D);
      mma(wa, xa, s);
      s += D;
      if (s >= s1) break;
      if (s + D < s1) load(wa, xa, s + D);
      mma(wb, xb, s);
      s += D;
    }
  }

  // Writes this wavefront's partial tile to LDS: red[((wave*RT + rt)*TT + tt)*64 + lane].
  __device__ __forceinline__ void stash(f32x4* red) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) red[((wave * RT + rt) * TT + tt) * 64 + lane] = acc[rt][tt];
  }

  // Sum over wavefronts, in wavefront (= K) order, of quad q < kQuads.
  __device__ static __forceinline__ f32x4 gather(const f32x4* red, int q) {
    f32x4 s = red[q];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red[w * kQuads + q];
    return s;
  }

  // Token and first row (relative to row0) of quad q.
  __device__ static __forceinline__ void quad_coords(int q, int& m, int& r) {
    const int rt = q / (TT * 64), tt = (q / 64) % TT, ln = q & 63;
    m = tt * 16 + (ln & 15);
    r = rt * 16 + 4 * (ln >> 4);
  }
};

// Rows of W per workgroup for N output rows: spread N over 256 workgroups (one
// per compute unit), a multiple of 4, at most 32 (two 16-row MFMA tiles).
__host__ __device__ inline int gemm_rows_per_wg(int N) {
  int r = (N + 255) / 256;
  r = (r + 3) & ~3;
  if (r < 4) r = 4;
  if (r > 32) r = 32;
  return r;
}

// The epilogue of quad q: rows r .. r+3 of token m, stored as two bf16 pairs;
// the row count of a workgroup is even, so each pair is all-in or all-out.
__device__ __forceinline__ void store_quad_pairs(uint16_t* row, int r, int rows, u32x2 v) {
  if (r < rows) *reinterpret_cast<unsigned*>(row + r) = v.x;
  if (r + 2 < rows) *reinterpret_cast<unsigned*>(row + r + 2) = v.y;
}

}  // namespace attnres
