// Standalone weight-stationary skinny GEMM (vLLM gemm.ws_gemm page, WsGemm):
// y = bf16(x W^T) with -0.0 stored as +0.0 (positive_zero).
#include "gemm.hpp"
#include "launch.hpp"

namespace attnres {

template <int RT, int TT>
__global__ __launch_bounds__(512) void wsgemm_kernel(GemmParams p, int R) {
  using C = GemmLdsFor<RT, TT>;
  static_assert(C::NT == 512, "launch bounds");
  __shared__ __attribute__((aligned(16))) char lds[C::kLdsBytes];
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // reused once the ring is drained
  const int row0 = blockIdx.x * R;
  const int rows = min(R, p.N - row0);
  C core;
  core.start(p.x, p.ldx, p.W, p.ldw, p.M, 0, p.K, row0, rows, lds);
  core.finish();
  core.stash(red);
  lds_barrier();
  for (int q = threadIdx.x; q < C::kQuads; q += C::NT) {
    int m, r;
    C::quad_coords(q, m, r);
    if (m < p.M && r < rows) {
      const f32x4 s = C::gather(red, q);
      const u32x2 v = {positive_zero(pack2(s.x, s.y)), positive_zero(pack2(s.z, s.w))};
      store_quad_pairs(p.y + (size_t)m * p.ldy + row0, r, rows, v);
    }
  }
}

template <int RT, int TT>
static hipError_t go(const GemmParams& p, int R, hipStream_t stream) {
  const int grid = (p.N + R - 1) / R;
  hipLaunchKernelGGL((wsgemm_kernel<RT, TT>), dim3(grid), dim3(GemmLdsFor<RT, TT>::NT), 0, stream, p, R);
  return hipGetLastError();
}

hipError_t launch_wsgemm(const GemmParams& p, hipStream_t stream) {
  const int R = gemm_rows_per_wg(p.N);
  const int tt = (p.M + 15) / 16;
  if (R > 16) {
    switch (tt) {
      case 1: return go<2, 1>(p, R, stream);
      case 2: return go<2, 2>(p, R, stream);
      case 3: return go<2, 3>(p, R, stream);
      default: return go<2, 4>(p, R, stream);
    }
  }
  switch (tt) {
    case 1: return go<1, 1>(p, R, stream);
    case 2: return go<1, 2>(p, R, stream);
    case 3: return go<1, 3>(p, R, stream);
    default: return go<1, 4>(p, R, stream);
  }
}

}  // namespace attnres
