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
//     then it signals `arrive`;
//   * workgroup t < M also owns token t's AttnRes: while the first stage of its
//     W loads is in flight it runs pre() on the token's saved blocks (results in
//     LDS); after its own signal it waits until every workgroup has arrived,
//     reads the token's full new prefix back and runs post().
// Only the owners wait, and they wait on workgroups that never wait, so the
// grid drains whatever the residency. The last owner to pass the wait resets
// the two counters, leaving the workspace zero for the next call.
//
// Hand-off without cache maintenance: the new prefix columns are stored with
// device-scope stores; each wavefront waits for its stores to complete
// (s_waitcnt vmcnt(0)) before the workgroup barrier that precedes the
// counter increment, and the owner reads the columns back with device-scope
// loads after it has seen the counter reach G (and invalidated its caches once).
// No L2 write-back is needed: nothing else the owner reads was written in this
// launch.
#include "gemm.hpp"
#include "launch.hpp"

namespace attnres {

#ifndef FUSED_D
#define FUSED_D(TT) ((TT) == 1 ? 4 : (TT) == 2 ? 4 : 2)
#endif

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

  // First stage of this workgroup's W and x loads goes out before anything else.
  C core;
  core.start(f.x, f.ldx, f.W, f.ldw, M, f.K, row0, rows);

  // ---- owner: pre() of token g, results to LDS --------------------------------
  // Two passes over the saved blocks keep the register footprint small while the
  // first W stage is held: the statistics pass, then (after the reduction) the
  // mixture pass, whose block reads hit in L2.
  PreScalars pre = {0.0f, 0.0f};
  u32x4 gq[NCH];
  if (owner) {
    const uint16_t* tok_blocks = a.blocks + (size_t)g * a.bst_t;
    float ps[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) ps[k] = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + j * NT;
      const bool valid = c < CH;
      const size_t col = (size_t)c * 8;
      gq[j] = valid ? ld16(a.out_norm + col) : zero;
      float w[8];
      if (valid) {
        weights8(a, c, w);
        f32x4* pw = reinterpret_cast<f32x4*>(lds_w + c * 8);
        pw[0] = f32x4{w[0], w[1], w[2], w[3]};
        pw[1] = f32x4{w[4], w[5], w[6], w[7]};
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.0f;
      }
#pragma unroll
      for (int b = 0; b < kMaxBlocks; ++b) {
        if (b < a.nb && valid) {
          float v[8];
          unpack8(ld16(tok_blocks + b * a.bst_b + col), v);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            ps[b] = __builtin_fmaf(v[i], v[i], ps[b]);
            ps[8 + b] = __builtin_fmaf(v[i], w[i], ps[8 + b]);
          }
        }
      }
    }
    if (a.nb > 0) {
      wg_sum<16, NW>(ps, lds_pre);
      float lg[kMaxBlocks], e[kMaxBlocks];
#pragma unroll
      for (int b = 0; b < kMaxBlocks; ++b) lg[b] = ps[8 + b] * rstd(ps[b], a.inv_h, a.eps);
      float m = lg[0];
#pragma unroll
      for (int b = 1; b < kMaxBlocks; ++b)
        if (b < a.nb) m = fmaxf(m, lg[b]);
      float S = 0.0f;
#pragma unroll
      for (int b = 0; b < kMaxBlocks; ++b) {
        e[b] = b < a.nb ? exp_fast(lg[b] - m) : 0.0f;
        S += e[b];
      }
      pre.maxl = m;
      pre.S = S;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = tid + j * NT;
        if (c < CH) {
          const size_t col = (size_t)c * 8;
          float mix[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) mix[i] = 0.0f;
#pragma unroll
          for (int b = 0; b < kMaxBlocks; ++b) {
            if (b < a.nb) {
              float v[8];
              unpack8(ld16(tok_blocks + b * a.bst_b + col), v);
#pragma unroll
              for (int i = 0; i < 8; ++i) mix[i] = __builtin_fmaf(e[b], v[i], mix[i]);
            }
          }
          f32x4* pm = reinterpret_cast<f32x4*>(lds_mix + c * 8);
          pm[0] = f32x4{mix[0], mix[1], mix[2], mix[3]};
          pm[1] = f32x4{mix[4], mix[5], mix[6], mix[7]};
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = tid + j * NT;
        if (c < CH) {
          f32x4* pm = reinterpret_cast<f32x4*>(lds_mix + c * 8);
          pm[0] = pm[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
  }

  // ---- GEMM share: rows [row0, row0 + rows) for all M tokens ---------------------
  core.finish();
  core.stash(red);
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
    st8_device(a.prefix + (size_t)qm * a.ld_prefix + col, nv);  // read back by owner qm
    if (a.aux) st8(a.aux + (size_t)qm * a.ld_aux + col, nv);
    if (a.write >= a.nb) st8(a.blocks + qm * a.bst_t + a.write * a.bst_b + col, nv);
  }

  // ---- hand-off: publish this workgroup's columns ---------------------------------
  wait_vmem();
  __syncthreads();
  if (tid == 0) __hip_atomic_fetch_add(&f.sync->arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!owner) return;

  if (tid == 0) {
    while (__hip_atomic_load(&f.sync->arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)G)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();

  // ---- owner: post() of token g ------------------------------------------------------
  const int t = g;
  u32x4 nbits[NCH];
  float nw[NCH][8], w[NCH][8], mix[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * NT;
    if (c < CH) {
      const uint16_t* src = a.prefix + (size_t)t * a.ld_prefix + (size_t)c * 8;
      const u32x2 lo = ld8_device(src), hi = ld8_device(src + 4);
      nbits[j] = u32x4{lo.x, lo.y, hi.x, hi.y};
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
  constexpr int D = FUSED_D(TT);
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
