// Standalone weight-stationary skinny GEMM (vLLM gemm.ws_gemm page, WsGemm):
// y = bf16(x W^T) with -0.0 stored as +0.0 (positive_zero); optionally with
// the MoE-front epilogue of WsGemm.epilogue (router rows as FP32 words,
// latent rows as bf16, the padding rows between dropped).
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
      if (!p.moe) {
        store_quad_pairs<false>(p.y + (size_t)m * p.ldy + row0, r, rows, v);
      } else {
        // valid and split are multiples of 8 and a quad's four rows start at
        // a multiple of 4: the whole quad falls in one shard
        const int c = row0 + r;
        uint16_t* orow = p.y + (size_t)m * p.ldy;
        if (c < p.valid) {  // router shard: FP32 words, -0.0 stored as +0.0
          unsigned* dst = reinterpret_cast<unsigned*>(orow + p.router_base + 2 * (p.slot + c));
          const u32x4 w = __builtin_bit_cast(u32x4, s);
          __builtin_nontemporal_store(w.x == kMailboxSentinel ? 0u : w.x, dst);
          __builtin_nontemporal_store(w.y == kMailboxSentinel ? 0u : w.y, dst + 1);
          __builtin_nontemporal_store(w.z == kMailboxSentinel ? 0u : w.z, dst + 2);
          __builtin_nontemporal_store(w.w == kMailboxSentinel ? 0u : w.w, dst + 3);
        } else if (c >= p.split) {  // latent shard: bf16 at base + c - split
          store_quad_pairs<false>(orow + p.base + (row0 - p.split), r, rows, v);
        }
      }
    }
  }
}

// Split K for more than 32 tokens (wsgemm_run_ws): S workgroups share each
// 64-row group, workgroup q streaming the q-th contiguous part of K. Every
// compute unit then reads 1/S of x next to its 64 rows of W, instead of all of
// x next to 16 rows (at M = 64 x would fill four fifths of the LDS ring). Parts
// 0 .. S-2 store their FP32 partial products in the workspace (the
// sentinel-armed hand-off of the fused call; stored zeros are +0.0, so no
// partial equals the sentinel) and finish; part S-1 polls them, adds the parts
// in part order (its own last), re-arms the words, rounds and writes y 16
// bytes at a time. Only the last part waits, and only on lower workgroup ids;
// a part that gives up flags the workspace header (its results are invalid),
// and a call on a flagged workspace writes nothing at all.
// Up to 128 tokens (eight 16-token tiles) stream through one pass: W is read
// once for all of them (the pages' token groups serve the same end).
// S (2 or 4) is a run-time argument: hipcc emitted the host launch stub of
// only one of two kernel instantiations that differed in nothing but S.
constexpr int kMaxSplit = 4;
template <int TT>
__global__ __launch_bounds__(512) void wsgemm_split_kernel(GemmParams p, unsigned* partials,
                                                           FusedWorkspace* ws, int ng, int kpart,
                                                           int S) {
  using C = GemmLdsSplit<TT>;
  static_assert(C::NT == 512, "launch bounds");
  static_assert(C::NP * C::kQuads * 16 + TT * 16 * kSplitRows * 2 <= C::kLdsBytes, "y tile fits");
  constexpr int QPT = (C::kQuads + C::NT - 1) / C::NT;
  __shared__ __attribute__((aligned(16))) char lds[C::kLdsBytes];
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // reused once the ring is drained
  const int g = blockIdx.x, tid = threadIdx.x;
  const int q = g / ng, rg = g - q * ng;  // part of K, row group
  const int row0 = rg * kSplitRows;
  const int rows = min(kSplitRows, p.N - row0);
  const int kbeg = q * kpart;
  const int klen = max(0, min(kpart, p.K - kbeg));
  // nonzero: an earlier call on this workspace gave up a wait, so this call
  // writes nothing (read by thread 0, used by the workgroup after a barrier)
  __shared__ unsigned lds_flag;
  const unsigned flag0 =
      tid == 0 ? __hip_atomic_load(&ws->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  int qm[QPT], qr[QPT];
  bool qv[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int qq = tid + i * C::NT;
    qm[i] = qr[i] = 0;
    qv[i] = false;
    if (qq < C::kQuads) {
      C::quad_coords(qq, qm[i], qr[i]);
      qv[i] = qm[i] < p.M && qr[i] < rows;
    }
  }
  {
    C core;
    core.start(p.x, p.ldx, p.W, p.ldw, p.M, kbeg, klen, row0, rows, lds, rg);
    core.finish();
    core.stash(red);
  }
  if (tid == 0) lds_flag = flag0;
  lds_barrier();
  if (lds_flag) return;  // the whole workgroup: the same LDS word after the barrier
  f32x4 s[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) s[i] = qv[i] ? C::gather(red, tid + i * C::NT) : f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t part =
      __builtin_amdgcn_make_buffer_rsrc(partials, 0, (S - 1) * ng * C::kQuads * 16, kBufferDword3);
  if (q < S - 1) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      if (qv[i]) {  // +0.0 for a zero, so no stored word equals the sentinel
        u32x4 v = __builtin_bit_cast(u32x4, s[i]);
        v.x = v.x == kMailboxSentinel ? 0u : v.x;
        v.y = v.y == kMailboxSentinel ? 0u : v.y;
        v.z = v.z == kMailboxSentinel ? 0u : v.z;
        v.w = v.w == kMailboxSentinel ? 0u : v.w;
        __builtin_amdgcn_raw_buffer_store_b128(
            v, part, ((q * ng + rg) * C::kQuads + tid + i * C::NT) * 16, 0, kCacheSC1);
      }
    }
    return;
  }
  // the last part: collect the others (as the fused call's owners poll)
  unsigned pending = 0;
#pragma unroll
  for (int j = 0; j < kMaxSplit - 1; ++j)
#pragma unroll
    for (int i = 0; i < QPT; ++i)
      if (j < S - 1 && qv[i]) pending |= 1u << (j * QPT + i);
  f32x4 got[kMaxSplit - 1][QPT];
#pragma unroll
  for (int j = 0; j < kMaxSplit - 1; ++j)
#pragma unroll
    for (int i = 0; i < QPT; ++i) got[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int spin = 0; pending != 0; ++spin) {
    u32x4 r[kMaxSplit - 1][QPT];
#pragma unroll
    for (int j = 0; j < kMaxSplit - 1; ++j)
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const unsigned off = (unsigned)((j * ng + rg) * C::kQuads + tid + i * C::NT) * 16u;
        r[j][i] = __builtin_amdgcn_raw_buffer_load_b128(
            part, (pending & (1u << (j * QPT + i))) ? off : kBufferOff, 0, kCacheSC1);
      }
#pragma unroll
    for (int j = 0; j < kMaxSplit - 1; ++j)
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const unsigned bit = 1u << (j * QPT + i);
        const u32x4 v = r[j][i];
        if ((pending & bit) && v.x != kMailboxSentinel && v.y != kMailboxSentinel &&
            v.z != kMailboxSentinel && v.w != kMailboxSentinel) {
          got[j][i] = __builtin_bit_cast(f32x4, v);
          pending &= ~bit;
        }
      }
    if (pending == 0) break;
    if (spin >= kSpinLimit) {  // gave up: flag the workspace (results invalid)
      __hip_atomic_store(&ws->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // y (rounded, -0.0 -> +0.0) of every quad into an LDS tile [token][64 rows]
  unsigned* tile = reinterpret_cast<unsigned*>(lds + C::NP * C::kQuads * 16);
  const u32x4 sent = {kMailboxSentinel, kMailboxSentinel, kMailboxSentinel, kMailboxSentinel};
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    if (qv[i]) {
      f32x4 t = got[0][i];
#pragma unroll
      for (int j = 1; j < kMaxSplit - 1; ++j)
        if (j < S - 1) t += got[j][i];
      t += s[i];
#pragma unroll
      for (int j = 0; j < kMaxSplit - 1; ++j)
        if (j < S - 1)
          __builtin_amdgcn_raw_buffer_store_b128(
              sent, part, ((j * ng + rg) * C::kQuads + tid + i * C::NT) * 16, 0, kCacheSC1);
      unsigned* t2 = tile + qm[i] * (kSplitRows / 2) + (qr[i] >> 1);
      t2[0] = positive_zero(pack2(t.x, t.y));
      t2[1] = positive_zero(pack2(t.z, t.w));
    }
  }
  lds_barrier();
  for (int it = tid; it < p.M * 8; it += C::NT) {  // 16 bytes (8 rows) of one token each
    const int om = it >> 3, oj = it & 7;
    if (8 * oj < rows)
      st16_nt(p.y + (size_t)om * p.ldy + row0 + 8 * oj,
           *reinterpret_cast<const u32x4*>(tile + om * (kSplitRows / 2) + 4 * oj));
  }
}

// The prepared layout of W (see packed_bytes in launch.hpp): thread i writes
// the 16-byte piece at position j = i % 16 of row n = (i / 16) % N in plane
// i / (16 N), which holds piece j ^ (n & 15) of that row's plane, or zeros
// past K (K is a multiple of 8, so a piece is all in or all out).
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                   int N, int K, uint16_t* __restrict__ Wp,
                                                   size_t pieces) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < pieces;
       i += (size_t)gridDim.x * blockDim.x) {
    const int j = (int)(i & 15);
    const size_t rn = i >> 4;
    const int n = (int)(rn % (size_t)N);
    const size_t plane = rn / (size_t)N;
    const size_t k = plane * 128 + (size_t)(8 * (j ^ (n & 15)));
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k < (size_t)K) v = ld16(W + (size_t)n * ldw + k);
    *reinterpret_cast<u32x4*>(Wp + (plane * N + n) * 128 + 8 * j) = v;
  }
}

hipError_t launch_pack_weights(const uint16_t* W, int64_t ldw, int N, int K, uint16_t* Wp,
                               hipStream_t stream) {
  const size_t pieces = packed_bytes(N, K) / 16;
  size_t blocks = (pieces + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, ldw, N, K, Wp,
                     pieces);
  return hipGetLastError();
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

template <int TT>
static hipError_t go_split(const GemmParams& p, unsigned* partials, FusedWorkspace* ws, int ng,
                           int S, hipStream_t stream) {
  using C = GemmLdsSplit<TT>;
  const int kpart = ((p.K + S - 1) / S + C::KE - 1) / C::KE * C::KE;  // whole chunks per part
  hipLaunchKernelGGL((wsgemm_split_kernel<TT>), dim3(S * ng), dim3(C::NT), 0, stream, p, partials,
                     ws, ng, kpart, S);
  return hipGetLastError();
}

bool wsgemm_ws_splits(int M, int N, int K, int compute_units) {
  const int ng = (N + kSplitRows - 1) / kSplitRows;
  return M > 32 && 2 * ng <= compute_units && K >= 256;
}

hipError_t launch_wsgemm_ws(const GemmParams& p, void* workspace, int compute_units,
                            hipStream_t stream) {
  const int tt = (p.M + 15) / 16;
  const int ng = (p.N + kSplitRows - 1) / kSplitRows;
  const int S = kMaxSplit * ng <= compute_units ? kMaxSplit : 2 * ng <= compute_units ? 2 : 1;
  if (!wsgemm_ws_splits(p.M, p.N, p.K, compute_units)) return launch_wsgemm(p, stream);
  FusedWorkspace* ws = static_cast<FusedWorkspace*>(workspace);
  unsigned* partials =
      reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + kWorkspaceHeader);
  switch (tt) {
    case 3: return go_split<3>(p, partials, ws, ng, S, stream);
    case 4: return go_split<4>(p, partials, ws, ng, S, stream);
    case 5: return go_split<5>(p, partials, ws, ng, S, stream);
    case 6: return go_split<6>(p, partials, ws, ng, S, stream);
    case 7: return go_split<7>(p, partials, ws, ng, S, stream);
    default: return go_split<8>(p, partials, ws, ng, S, stream);
  }
}

}  // namespace attnres
