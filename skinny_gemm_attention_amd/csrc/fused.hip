// The fused decode step: o-projection (weight-stationary GEMM) + AttnRes, one
// launch (vLLM oproj.prepared page: the o-projection output is the AttnRes
// delta of the same layer; attn_res.kernel page: ClusterAttnRes; gemm.ws_gemm
// page: WsGemm).
//
// Roles inside one grid of G = max(ceil(H / R), M) workgroups:
//   * every workgroup g owns rows [g R, g R + R) of W (the GEMM) and, for all M
//     tokens, the matching columns of the new prefix: it rounds its y columns to
//     bf16 (-0.0 -> +0.0), forms new = bf16(prefix + y) (or y) and stores new
//     to prefix, aux and, when the written slot is not scored, the block slot;
//     then it signals `arrive` (release);
//   * workgroup t < M also owns token t's AttnRes: before its GEMM share it runs
//     pre() on the token's saved blocks (off the critical path, results in
//     LDS); after its own signal it waits until every workgroup has arrived
//     (acquire), reads the token's full new prefix back and runs post().
// Only the owners wait, and they wait on workgroups that never wait, so the
// grid drains whatever the residency. The last owner to pass the wait resets
// the two counters, leaving the workspace zero for the next call.
#include "gemm.hpp"
#include "launch.hpp"

namespace attnres {

template <int RT, int TT, int NW, int D>
__global__ __launch_bounds__(NW * 64) void fused_kernel(FusedParams f, int R, int G) {
  using C = GemmCore<RT, TT, NW, D>;
  constexpr int NT = NW * 64;
  constexpr int NCH = TokenShape<NT>::NCH;
  __shared__ f32x4 red[NW * C::kQuads];
  __shared__ float lds_mix[kMaxH], lds_w[kMaxH];
  __shared__ float lds_pre[NW * 16], lds_post[NW * 4], lds_fin[NW];

  const AttnParams& a = f.a;
  const int g = blockIdx.x, tid = threadIdx.x, CH = a.H >> 3;
  const int M = a.T;
  const bool owner = g < M;
  const int row0 = g * R;
  const int rows = row0 < a.H ? min(R, a.H - row0) : 0;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // This thread's quad of the GEMM epilogue and its old prefix (prefetched).
  int qm = 0, qr = 0;
  bool qvalid = false;
  u32x2 qprefix = {0u, 0u};
  if (tid < C::kQuads) {
    C::quad_coords(tid, qm, qr);
    qvalid = qm < M && qr < rows;
    if (qvalid && a.has_delta) qprefix = ld8(a.prefix + (size_t)qm * a.ld_prefix + row0 + qr);
  }

  // ---- owner: pre() of token g, results to LDS --------------------------------
  PreScalars pre = {0.0f, 0.0f};
  u32x4 gq[NCH];
  if (owner) {
    u32x4 vb[kMaxBlocks][NCH];
    float w[NCH][8];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + j * NT;
      const bool valid = c < CH;
      const size_t col = (size_t)c * 8;
#pragma unroll
      for (int b = 0; b < kMaxBlocks; ++b)
        vb[b][j] = (valid && b < a.nb) ? ld16(a.blocks + g * a.bst_t + b * a.bst_b + col) : zero;
      gq[j] = valid ? ld16(a.out_norm + col) : zero;
      if (valid) {
        weights8(a, c, w[j]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[j][i] = 0.0f;
      }
    }
    float mix[NCH][8];
    if (a.nb > 0) {
      float ps[16];
      pre_partials(vb, w, a.nb, ps);
      wg_sum<16, NW>(ps, lds_pre);
      pre = pre_finish(ps, vb, a.nb, a.eps, a.inv_h, mix);
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) mix[j][i] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + j * NT;
      if (c < CH) {
        f32x4* pm = reinterpret_cast<f32x4*>(lds_mix + c * 8);
        f32x4* pw = reinterpret_cast<f32x4*>(lds_w + c * 8);
        pm[0] = f32x4{mix[j][0], mix[j][1], mix[j][2], mix[j][3]};
        pm[1] = f32x4{mix[j][4], mix[j][5], mix[j][6], mix[j][7]};
        pw[0] = f32x4{w[j][0], w[j][1], w[j][2], w[j][3]};
        pw[1] = f32x4{w[j][4], w[j][5], w[j][6], w[j][7]};
      }
    }
  }

  // ---- GEMM share: rows [row0, row0 + rows) for all M tokens ---------------------
  {
    f32x4 acc[RT][TT];
    C::accumulate(f.x, f.ldx, f.W, f.ldw, M, f.K, row0, rows, acc);
    C::stash(red, acc);
  }
  __syncthreads();
  if (qvalid) {
    const f32x4 s = C::gather(red, tid);
    const unsigned y01 = positive_zero(pack2(s.x, s.y)), y23 = positive_zero(pack2(s.z, s.w));
    u32x2 nv;
    if (a.has_delta) {
      nv.x = pack2(add_round_odd(bf_lo(qprefix.x), bf_lo(y01)), add_round_odd(bf_hi(qprefix.x), bf_hi(y01)));
      nv.y = pack2(add_round_odd(bf_lo(qprefix.y), bf_lo(y23)), add_round_odd(bf_hi(qprefix.y), bf_hi(y23)));
    } else {
      nv = u32x2{y01, y23};
    }
    const size_t col = (size_t)(row0 + qr);
    st8(a.prefix + (size_t)qm * a.ld_prefix + col, nv);
    if (a.aux) st8(a.aux + (size_t)qm * a.ld_aux + col, nv);
    if (a.write >= a.nb) st8(a.blocks + qm * a.bst_t + a.write * a.bst_b + col, nv);
  }

  // ---- hand-off: publish this workgroup's columns ---------------------------------
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) __hip_atomic_fetch_add(&f.sync->arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!owner) return;

  if (tid == 0) {
    while (__hip_atomic_load(&f.sync->arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)G)
      __builtin_amdgcn_s_sleep(1);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- owner: post() of token g ------------------------------------------------------
  const int t = g;
  u32x4 nbits[NCH];
  float nw[NCH][8], w[NCH][8], mix[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * NT;
    if (c < CH) {
      nbits[j] = ld16(a.prefix + (size_t)t * a.ld_prefix + (size_t)c * 8);
      const f32x4* pm = reinterpret_cast<const f32x4*>(lds_mix + c * 8);
      const f32x4* pw = reinterpret_cast<const f32x4*>(lds_w + c * 8);
      const f32x4 m0 = pm[0], m1 = pm[1], w0 = pw[0], w1 = pw[1];
      mix[j][0] = m0.x; mix[j][1] = m0.y; mix[j][2] = m0.z; mix[j][3] = m0.w;
      mix[j][4] = m1.x; mix[j][5] = m1.y; mix[j][6] = m1.z; mix[j][7] = m1.w;
      w[j][0] = w0.x; w[j][1] = w0.y; w[j][2] = w0.z; w[j][3] = w0.w;
      w[j][4] = w1.x; w[j][5] = w1.y; w[j][6] = w1.z; w[j][7] = w1.w;
    } else {
      nbits[j] = zero;
#pragma unroll
      for (int i = 0; i < 8; ++i) mix[j][i] = w[j][i] = 0.0f;
    }
    unpack8(nbits[j], nw[j]);
  }
  // every owner is past the wait once `done` reaches M: the last one resets
  if (tid == 0) {
    const unsigned d = __hip_atomic_fetch_add(&f.sync->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == (unsigned)M - 1u) {
      __hip_atomic_store(&f.sync->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&f.sync->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  float pp[4];
  post_partials(nw, w, mix, pp);
  wg_sum<4, NW>(pp, lds_post);
  if (a.write >= 0 && a.write < a.nb) {  // a scored slot: written after pre() read it
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + j * NT;
      if (c < CH) st16(a.blocks + t * a.bst_t + a.write * a.bst_b + (size_t)c * 8, nbits[j]);
    }
  }
  finish_out<NT, NCH>(a, t, pre, pp, nw, mix, gq, lds_fin);
}

template <int RT, int TT>
static hipError_t go(const FusedParams& p, int R, hipStream_t stream) {
  constexpr int NW = 8;
  constexpr int D = TT == 1 ? 8 : TT == 2 ? 6 : TT == 3 ? 4 : 3;
  const int gemm_wgs = (p.a.H + R - 1) / R;
  const int G = gemm_wgs > p.a.T ? gemm_wgs : p.a.T;
  hipLaunchKernelGGL((fused_kernel<RT, TT, NW, D>), dim3(G), dim3(NW * 64), 0, stream, p, R, G);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedParams& p, hipStream_t stream) {
  const int R = gemm_rows_per_wg(p.a.H);
  const int tt = (p.a.T + 15) / 16;
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
