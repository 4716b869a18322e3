// AttnRes with the delta given as a tensor (vLLM attn_res.kernel page,
// ClusterAttnRes with a tensor delta): one workgroup per token.
//
// Every load of the token is issued up front (saved blocks, norm, query,
// out_norm, delta, old prefix), so one DRAM round trip covers the whole row
// set; the two (final boundary: three) 7168-wide sums are fixed-order
// workgroup reductions.
//
// STATS: post() on carried saved-block statistics (the state ClusterAttnRes
// keeps between pre and post: the mixture row and maximum / exp_sum), as the
// fused kernel stores them for the next layer (oproj.prepared page,
// PreparedOproj.bind_ahead). The saved blocks are then not read; everything
// after pre is the same code, so given the statistics that pre would have
// formed, the results are the same bits.
#include "launch.hpp"

namespace attnres {

template <int NT, bool STATS>
__global__ __launch_bounds__(NT) void attnres_kernel(AttnParams a) {
  constexpr int NW = TokenShape<NT>::NW, NCH = TokenShape<NT>::NCH;
  __shared__ float lds_pre[wg_sum_lds<16, NW>], lds_post[wg_sum_lds<4, NW>],
      lds_fin[wg_sum_lds<1, NW>];
  const int t = blockIdx.x, tid = threadIdx.x, CH = a.H >> 3;
  // Every load of the token is a raw buffer load issued before any result is
  // used: a saved block past nb, an unused tensor (num_records 0) or a lane
  // past the row (an offset past the end) reads zeros without touching
  // memory. (Loads written as `cond ? ld16(p) : 0` became branches whose
  // register copies made the compiler wait for every earlier load in the
  // middle of the sequence.) The token's saved blocks, delta and old prefix
  // are read once: non-temporal (measured at T = 256: 13.5 -> 11.4 us at
  // nb = 8, 5.76 -> 5.38 us at nb = 0). The gains, read by every workgroup,
  // and the carried mixture keep the default policy (a non-temporal mixture
  // read made attnres_post_run slower, 6.13 -> 6.58 us).
  const int H2 = a.H * 2;
  auto rsrc = [](const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferDword3);
  };
  const __amdgpu_buffer_rsrc_t r_norm = rsrc(a.norm, H2), r_query = rsrc(a.query, H2),
                               r_gain = rsrc(a.out_norm, H2),
                               r_delta = rsrc(a.delta + (size_t)t * a.ld_delta, H2),
                               r_prefix = rsrc(a.prefix + (size_t)t * a.ld_prefix,
                                               a.has_delta ? H2 : 0),
                               r_smix = rsrc(STATS ? a.smix + (size_t)t * a.ld_smix : nullptr,
                                             (STATS && a.nb > 0) ? 2 * H2 : 0);
  u32x4 vb[kMaxBlocks][NCH], g[NCH], d[NCH], p[NCH], sm[NCH][2], nq[NCH][2];
  unsigned off[NCH], off4[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * NT;
    const bool valid = c < CH;
    off[j] = valid ? (unsigned)c * 16u : kBufferOff;    // bf16 rows
    off4[j] = valid ? (unsigned)c * 32u : kBufferOff;   // FP32 rows
    nq[j][0] = __builtin_amdgcn_raw_buffer_load_b128(r_norm, off[j], 0, 0);
    nq[j][1] = __builtin_amdgcn_raw_buffer_load_b128(r_query, off[j], 0, 0);
  }
  // what pre needs first: every saved block of both chunks, then the rest
  // (loads complete in issue order, so pre then waits for no delta, prefix or
  // gain: 1-5% faster at T = 256 for nb >= 2)
#pragma unroll
  for (int j = 0; j < NCH; ++j)
#pragma unroll
    for (int b = 0; b < kMaxBlocks; ++b) {
      const bool live = !STATS && b < a.nb;  // blocks may be NULL when nb == 0
      const __amdgpu_buffer_rsrc_t r_blk =
          rsrc(live ? a.blocks + (size_t)t * a.bst_t + (size_t)b * a.bst_b : a.blocks, live ? H2 : 0);
      vb[b][j] = __builtin_amdgcn_raw_buffer_load_b128(r_blk, off[j], 0, kCacheNTLoad);
    }
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    sm[j][0] = __builtin_amdgcn_raw_buffer_load_b128(r_smix, off4[j], 0, 0);
    sm[j][1] = __builtin_amdgcn_raw_buffer_load_b128(r_smix, off4[j] == kBufferOff ? kBufferOff : off4[j] + 16u, 0, 0);
    g[j] = __builtin_amdgcn_raw_buffer_load_b128(r_gain, off[j], 0, 0);
    d[j] = __builtin_amdgcn_raw_buffer_load_b128(r_delta, off[j], 0, kCacheNTLoad);
    p[j] = __builtin_amdgcn_raw_buffer_load_b128(r_prefix, off[j], 0, kCacheNTLoad);
  }
  float w[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    float n[8], q[8];
    unpack8(nq[j][0], n);
    unpack8(nq[j][1], q);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[j][i] = n[i] * q[i];  // exact: product of two bf16
  }

  // pre: saved-block statistics and the unnormalised mixture
  float mix[NCH][8];
  BlockStats pre = {0.0f, 0.0f};
  if (STATS) {
    if (a.nb > 0) {
      pre.anchor = a.sscal[2 * t];
      pre.total = a.sscal[2 * t + 1];
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 v = __builtin_bit_cast(f32x4, sm[j][h]);
        mix[j][4 * h] = v.x;
        mix[j][4 * h + 1] = v.y;
        mix[j][4 * h + 2] = v.z;
        mix[j][4 * h + 3] = v.w;
      }
  } else if (a.nb > 0) {
    float ps[16];
    pre_partials(vb, w, a.nb, ps);
    wg_sum<16, NW>(ps, lds_pre);
    pre = block_stats(ps, vb, a.nb, a.eps, a.inv_h, mix);
  } else {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) mix[j][i] = 0.0f;
  }

  // residual update: new = bf16(prefix + delta), or the delta itself
  u32x4 nbits[NCH];
  float nw[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (a.has_delta) {
      float pf[8], df[8];
      unpack8(p[j], pf);
      unpack8(d[j], df);
      nbits[j].x = pack2(add_bf16_exact(pf[0], df[0]), add_bf16_exact(pf[1], df[1]));
      nbits[j].y = pack2(add_bf16_exact(pf[2], df[2]), add_bf16_exact(pf[3], df[3]));
      nbits[j].z = pack2(add_bf16_exact(pf[4], df[4]), add_bf16_exact(pf[5], df[5]));
      nbits[j].w = pack2(add_bf16_exact(pf[6], df[6]), add_bf16_exact(pf[7], df[7]));
    } else {
      nbits[j] = d[j];
    }
    unpack8(nbits[j], nw[j]);
  }

  float pp[4];
  post_partials(nw, w, mix, pp);
  wg_sum<4, NW>(pp, lds_post);

  // state: the same bits go to prefix, aux and the written block slot
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + j * NT;
    if (c < CH) {
      const size_t col = (size_t)c * 8;
      st16_nt(a.prefix + t * a.ld_prefix + col, nbits[j]);
      if (a.aux) st16_nt(a.aux + t * a.ld_aux + col, nbits[j]);
      if (a.write >= 0) st16_nt(a.blocks + t * a.bst_t + a.write * a.bst_b + col, nbits[j]);
    }
  }

  float gg[NCH][8], ng[NCH][8], mg[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    unpack8(g[j], gg[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ng[j][i] = nw[j][i] * gg[j][i];
      mg[j][i] = mix[j][i] * gg[j][i];
    }
  }
  finish_out<NT, NCH, false>(a, t, out_coefs(a, pre, pp), nw, ng, mix, mg, gg, lds_fin);
}

hipError_t launch_attnres(const AttnParams& p, hipStream_t stream) {
  constexpr int NT = kTokenThreads;
  if (p.smix)
    hipLaunchKernelGGL((attnres_kernel<NT, true>), dim3(p.T), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attnres_kernel<NT, false>), dim3(p.T), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attnres
