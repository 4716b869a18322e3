// The fused decode step: o-projection (weight-stationary GEMM) + AttnRes, one
// launch (vLLM oproj.prepared page: the o-projection output is the AttnRes
// delta of the same layer; attn_res.kernel page: ClusterAttnRes; gemm.ws_gemm
// page: WsGemm).
//
// One grid of 512-thread workgroups, two roles:
//   * GEMM workgroups g < G each own rows [g R, g R + R) of W and, for all M
//     tokens, the matching columns of the new prefix: they round their y
//     columns to bf16 (-0.0 -> +0.0), form new = bf16(prefix + y) (or y), store
//     new to prefix, aux and, when the written slot is not scored, the block
//     slot, and post it to the token's mailbox row. They never wait.
//   * Owner workgroups G + o (o < NO) own tokens o and o + NO (one token up to
//     32 tokens, two beyond): they run pre() on each token's saved blocks
//     while the GEMM workgroups stream W (ClusterAttnRes.state: pre needs
//     nothing the GEMM produces), then collect each token's new prefix from
//     its mailbox row and run post().
// Beyond 32 tokens each 64-row group of W is streamed by two GEMM workgroups
// taking alternate 4 KB blocks of K; the first hands its FP32 partial
// products to the second (a higher id) through the same sentinel scheme, and
// the second forms and posts the new prefix.
// R (even, at most 32) is chosen so that G + NO fits the compute units (for
// H = 7168: 239 GEMM workgroups of 30 rows): the owners' saved-block reads then
// overlap the W stream on units of their own instead of extending it. Every
// wait is on a lower workgroup id (owners are the highest ids), so with
// workgroups dispatched in id order the grid drains whatever the residency.
//
// With look-ahead statistics (fused_ahead_kernel; oproj.prepared page,
// PreparedOproj.bind_ahead) the owners also form, from the saved blocks they
// already hold, the pre() state of the next layer's AttnRes (its norm, query
// and eps) and store it: mixture row and (anchor, weight total) per token.
//
// Mailbox hand-off (the sentinel scheme of the pages' Lamport mailboxes,
// oproj.prepared page and positive_zero on the gemm.ws_gemm page): every
// mailbox word holds the bf16 pair (+0.0, -0.0) between calls. A new-prefix
// pair never contains -0.0 (the delta's -0.0 is made +0.0 and a bf16 sum
// that is zero is +0.0), so a word differs from the sentinel exactly when its
// value has arrived. GEMM workgroups write each pair once with a device-scope
// (sc1) store; each owner thread polls its own 8-column chunks with
// device-scope loads, in a fixed chunk order, and re-arms them after reading
// (never earlier in the call: a word re-armed before its value is posted
// stays valid in the owner XCD's L2, where the polls can keep reading it; the
// next call polls after a kernel boundary, whose acquire drops such lines).
// One memory latency separates a store from its consumer; no counter, fence or
// cache write-back is involved. A spin limit bounds every wait: a workgroup
// that gives up records it in the workspace header and carries on to the end
// (every thread still reaches every barrier; that call's outputs are
// invalid). A call whose workspace header is already set writes nothing, so
// a flagged workspace stays unusable until it is re-armed: in a GEMM
// workgroup thread 0 reads the header as it starts and shares it at the
// barrier after the W stream, and the workgroup returns before its first
// store; in an owner each wavefront reads it as it starts, skips its
// look-ahead stores and returns before polling. (A wavefront that has ended
// no longer takes part in its workgroup's barriers. Returning before pre(),
// right after the first loads, made the compiler wait for every outstanding
// load before each LDS read of the W stream: 64 tokens, K = 8192, 30.7 -> 42.7 us.)
#include "gemm.hpp"
#include "launch.hpp"

namespace attnres {

constexpr int kMaxTokensPerOwner = 2;


template <bool SPLIT, int RT, int TT, bool PACKED>
struct FusedCore {
  using type = GemmLdsFor<RT, TT, PACKED>;
};
template <int RT, int TT, bool PACKED>
struct FusedCore<true, RT, TT, PACKED> {
  static_assert(RT * 16 == kSplitRows, "split-K row groups");
  using type = GemmLdsSplit<TT, PACKED>;
};

template <int RT, int TT, bool SPLIT, bool AHEAD, bool PACKED>
__device__ __forceinline__ void fused_body(const FusedParams& f, int R, int G, int NO) {
  constexpr int NT = kTokenThreads, NW = NT / 64;
  using C = typename FusedCore<SPLIT, RT, TT, PACKED>::type;
  // the GEMM role's outputs written through up to 32 tokens (one token,
  // K = 1024 and eight tokens, K = 4096: 0.15 and 0.42 us faster per step);
  // beyond, with four times the bytes per workgroup, non-temporal (written
  // through was 0.08 us slower at 64 tokens). The owners' output rows are
  // non-temporal at every size: their completion ends the step, and the L2
  // acknowledges a non-temporal store sooner (0.02-0.04 us per step).
  constexpr bool WT = !SPLIT;
  static_assert(C::NT == NT, "one workgroup shape for both roles");
  // tokens per owner: one up to 32 tokens, two beyond
  constexpr int KT = TT <= 2 ? 1 : kMaxTokensPerOwner;
  constexpr int NCH = TokenShape<NT>::NCH;
  constexpr bool kOne = KT == 1;
  struct Smem {
    char ring[C::kLdsBytes];  // GEMM role: chunk ring, then the K partials
  };
  __shared__ __attribute__((aligned(16))) Smem sm;
  f32x4* red = reinterpret_cast<f32x4*>(sm.ring);
  __shared__ float lds_pre[wg_sum_lds<(4 * KT > 16 ? 4 * KT : 16), NW>],
      lds_fin[wg_sum_lds<1, NW>];
  __shared__ unsigned lds_flag;  // GEMM role: thread 0's reading of the workspace flag

  const AttnParams& a = f.a;
  const int g = blockIdx.x, tid = threadIdx.x, CH = a.H >> 3;
  const int M = a.T;

  if (g < G) {
    // ---- GEMM role: rows [row0, row0 + rows) for all M tokens -----------------------
    // Nothing is outstanding here; the explicit wait tells the compiler so.
    // Its control flow joins the owner role's exit with this entry, and its
    // wait bookkeeping then carried the owner's loads into this role: a
    // vmcnt(0) before a fragment read of the ring (a memory round trip) that
    // came and went with unrelated owner-side changes.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) only
    // Split K: workgroup g < ng streams the even 4 KB blocks (16 chunks) of
    // the K range of row group g and hands its FP32 partials to workgroup
    // g + ng, which streams the odd blocks, adds the two (even part first)
    // and finishes the rows. (Measured at M = 64, K = 8192: 1% faster than
    // contiguous halves; alternating 256 B to 2 KB pieces was 6-10% slower.)
    // The first workgroup never waits; the second waits only on a lower
    // workgroup id.
    // nonzero: an earlier call on this workspace gave up a wait, so this call
    // writes nothing (read by thread 0, shared at the barrier after the ring)
    const unsigned flag0 =
        tid == 0 ? __hip_atomic_load(&f.ws->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    const bool second = SPLIT && g >= f.ng;
    const int rg = SPLIT ? (second ? g - f.ng : g) : g;
    const int row0 = rg * R;
    const int rows = min(R, a.H - row0);
    constexpr int kSplitBlock = 16;  // chunks per block of the alternation
    const int kbeg = second ? kSplitBlock * C::KE : 0;
    const int klen = second ? f.K - kSplitBlock * C::KE : f.K;
    const bool finisher = !SPLIT || second;
    constexpr int QPT = (C::kQuads + NT - 1) / NT;  // output quads per thread
    // split finisher: thread (token tid / 8, rows 8 (tid % 8) .. + 7) writes
    // the new prefix 16 bytes at a time
    const int om = tid >> 3, oj = tid & 7;
    const bool ov = SPLIT && second && om < M && 8 * oj < rows;
    u32x4 oprefix = {0u, 0u, 0u, 0u};
    if (ov && a.has_delta) oprefix = ld16(a.prefix + (size_t)om * a.ld_prefix + row0 + 8 * oj);
    int qm[QPT], qr[QPT];
    bool qv[QPT];
    u32x2 qprefix[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = tid + i * NT;
      qm[i] = qr[i] = 0;
      qprefix[i] = u32x2{0u, 0u};
      qv[i] = false;
      if (q < C::kQuads) {
        C::quad_coords(q, qm[i], qr[i]);
        qv[i] = qm[i] < M && qr[i] < rows;
        if (!SPLIT && qv[i] && a.has_delta) {
          const uint16_t* src = a.prefix + (size_t)qm[i] * a.ld_prefix + row0 + qr[i];
          qprefix[i].x = *reinterpret_cast<const unsigned*>(src);
          if (qr[i] + 2 < rows) qprefix[i].y = *reinterpret_cast<const unsigned*>(src + 2);
        }
      }
    }
    {
      C core;
      // (a prepared W is swept plane by plane by all workgroups together, so
      // its chunks are not rotated)
      core.start(f.x, f.ldx, f.W, f.ldw, M, kbeg, klen, row0, rows, sm.ring, SPLIT && !PACKED ? rg : 0,
                 SPLIT ? 2 : 1, SPLIT ? kSplitBlock : 1, PACKED ? f.wrows : 0);
      core.finish();
      core.stash(red);
    }
    if (tid == 0) lds_flag = flag0;
    lds_barrier();
    // the flag is read with the partials (one LDS round trip for both)
    const unsigned flag = lds_flag;
    f32x4 s[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) s[i] = qv[i] ? C::gather(red, tid + i * NT) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (flag) return;  // the whole workgroup: the same LDS word after the barrier
    if (SPLIT) {
      const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
          f.partials, 0, f.ng * C::kQuads * 16, kBufferDword3);
      if (!second) {
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
          if (qv[i]) {  // +0.0 for a zero, so no stored word equals the sentinel
            u32x4 v = __builtin_bit_cast(u32x4, s[i]);
            v.x = v.x == kMailboxSentinel ? 0u : v.x;
            v.y = v.y == kMailboxSentinel ? 0u : v.y;
            v.z = v.z == kMailboxSentinel ? 0u : v.z;
            v.w = v.w == kMailboxSentinel ? 0u : v.w;
            __builtin_amdgcn_raw_buffer_store_b128(v, part, (rg * C::kQuads + tid + i * NT) * 16, 0,
                                                   kCacheSC1);
          }
        }
        return;
      }
      // the first workgroup's partials: poll (as the owners poll the mailbox),
      // add, re-arm
      unsigned pending = 0;
#pragma unroll
      for (int i = 0; i < QPT; ++i)
        if (qv[i]) pending |= 1u << i;
      f32x4 first[QPT];
      for (int spin = 0; pending != 0; ++spin) {
        u32x4 r[QPT];
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
          const unsigned off = (unsigned)(rg * C::kQuads + tid + i * NT) * 16u;
          r[i] = __builtin_amdgcn_raw_buffer_load_b128(part, (pending & (1u << i)) ? off : kBufferOff,
                                                       0, kCacheSC1);
        }
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
          const u32x4 v = r[i];
          if ((pending & (1u << i)) && v.x != kMailboxSentinel && v.y != kMailboxSentinel &&
              v.z != kMailboxSentinel && v.w != kMailboxSentinel) {
            first[i] = __builtin_bit_cast(f32x4, v);
            pending &= ~(1u << i);
          }
        }
        if (pending == 0) break;
        if (spin >= kSpinLimit) {  // gave up: flag the workspace (results invalid)
          __hip_atomic_store(&f.ws->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int i = 0; i < QPT; ++i)
            if (pending & (1u << i)) first[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      // y (rounded, -0.0 -> +0.0) of every quad into an LDS tile [token][64 rows]
      unsigned* tile = reinterpret_cast<unsigned*>(sm.ring + C::NP * C::kQuads * 16);
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        if (qv[i]) {
          s[i] = first[i] + s[i];
          unsigned* t2 = tile + qm[i] * (kSplitRows / 2) + (qr[i] >> 1);
          t2[0] = positive_zero(pack2(s[i].x, s[i].y));
          t2[1] = positive_zero(pack2(s[i].z, s[i].w));
        }
      }
      lds_barrier();
      if (ov) {
        const u32x4 y = *reinterpret_cast<const u32x4*>(tile + om * (kSplitRows / 2) + 4 * oj);
        u32x4 nv = y;
        if (a.has_delta) {
          float pf[8], yf[8], r[8];
          unpack8(oprefix, pf);
          unpack8(y, yf);
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = add_bf16_exact(pf[e], yf[e]);
          nv = pack8(r);
        }
        const size_t col = (size_t)row0 + 8 * oj;
        const __amdgpu_buffer_rsrc_t mb =
            __builtin_amdgcn_make_buffer_rsrc(f.mailbox, 0, M * a.H * 2, kBufferDword3);
        __builtin_amdgcn_raw_buffer_store_b128(nv, mb, (unsigned)((size_t)om * a.H + col) * 2u, 0,
                                               kCacheSC1);  // collected by token om's owner
        st16<WT>(a.prefix + (size_t)om * a.ld_prefix + col, nv);
        if (a.aux) st16<WT>(a.aux + (size_t)om * a.ld_aux + col, nv);
        if (a.write >= a.nb) st16<WT>(a.blocks + om * a.bst_t + a.write * a.bst_b + col, nv);
      }
      // re-arm the first workgroup's partials after the stores the owners wait
      // for (before them, the mailbox posts queued behind 16 KB of re-arm
      // stores: 0.09 us slower at 64 tokens, K = 8192)
      const u32x4 sent = {kMailboxSentinel, kMailboxSentinel, kMailboxSentinel, kMailboxSentinel};
#pragma unroll
      for (int i = 0; i < QPT; ++i)
        if (qv[i])
          __builtin_amdgcn_raw_buffer_store_b128(sent, part, (rg * C::kQuads + tid + i * NT) * 16, 0,
                                                 kCacheSC1);
      return;
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      if (qv[i]) {
        const unsigned y01 = positive_zero(pack2(s[i].x, s[i].y)), y23 = positive_zero(pack2(s[i].z, s[i].w));
        u32x2 nv;
        if (a.has_delta) {
          nv.x = pack2(add_bf16_exact(bf_lo(qprefix[i].x), bf_lo(y01)),
                       add_bf16_exact(bf_hi(qprefix[i].x), bf_hi(y01)));
          nv.y = pack2(add_bf16_exact(bf_lo(qprefix[i].y), bf_lo(y23)),
                       add_bf16_exact(bf_hi(qprefix[i].y), bf_hi(y23)));
        } else {
          nv = u32x2{y01, y23};
        }
        unsigned* box = f.mailbox + (size_t)qm[i] * (a.H >> 1) + ((row0 + qr[i]) >> 1);
        st4_wt(box, nv.x);  // collected by token qm's owner
        if (qr[i] + 2 < rows) st4_wt(box + 1, nv.y);
        store_quad_pairs<WT>(a.prefix + (size_t)qm[i] * a.ld_prefix + row0, qr[i], rows, nv);
        if (a.aux) store_quad_pairs<WT>(a.aux + (size_t)qm[i] * a.ld_aux + row0, qr[i], rows, nv);
        if (a.write >= a.nb)
          store_quad_pairs<WT>(a.blocks + qm[i] * a.bst_t + a.write * a.bst_b + row0, qr[i], rows, nv);
      }
    }
    return;
  }

  // ---- owner role: tokens o, o + NO, ... --------------------------------------------
  const int o = g - G;
  int ntok = 0;
#pragma unroll
  for (int k = 0; k < KT; ++k)
    if (o + k * NO < M) ntok = k + 1;

  // nonzero: an earlier call on this workspace gave up a wait, so this call
  // writes nothing. Each wavefront reads it and returns as a whole before its
  // first store; a wavefront that has ended no longer takes part in the
  // workgroup's barriers, so the others never wait for it. (Taking its value
  // only after pre() was 0.07-0.15 us slower per step.)
  const unsigned flagw = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(&f.ws->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  float gg[NCH][8], w[NCH][8], w2[AHEAD ? NCH : 1][8];
  token_weights<NT, NCH>(a, w, gg);
  if constexpr (AHEAD) pair_weights<NT, NCH>(f.ah.norm, f.ah.query, a.H, w2);
  BlockStats pre[KT];
  // the mixtures of this thread's chunks stay in registers: with one token,
  // with mixture*gains beside them; with two, the mixtures alone (before,
  // parked in LDS: 64 tokens 0.23 us slower, the tail's partials and outputs
  // waiting for the reads)
  float mix1[kOne ? NCH : 1][8], mg1[kOne ? NCH : 1][8];
  float mixk[kOne ? 1 : KT][kOne ? 1 : NCH][8];
  float pm2[KT][NCH];  // per-chunk sums of mix^2 (the post partial that needs no new prefix)
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    pre[k] = BlockStats{0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      pm2[k][j] = 0.0f;
      if (!kOne)
#pragma unroll
        for (int i = 0; i < 8; ++i) mixk[kOne ? 0 : k][kOne ? 0 : j][i] = 0.0f;
    }
    if (k < ntok) {
      const int t = o + k * NO;
      float mix[NCH][8];
      if constexpr (AHEAD) {
        // the next layer's statistics over the same (launch-time) saved
        // blocks, stored for its post (oproj.prepared page, bind_ahead);
        // non-temporal (a later kernel reads them; plain stores cost about
        // 2 us at 64 tokens, and written through, the owner's polls behind
        // them waited for their slower completion: 1.1 us at one token)
        float mix2[NCH][8];
        BlockStats pre2;
        token_pre2<NT, NCH>(a, t, w, w2, f.ah.eps, mix, mix2, pre[k], pre2, lds_pre);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const int c = tid + j * NT;
          if (c < CH && !flagw) {
            float* dst = f.ah.mix + (size_t)t * f.ah.ld_mix + (size_t)c * 8;
            st16_nt(dst, __builtin_bit_cast(u32x4, f32x4{mix2[j][0], mix2[j][1], mix2[j][2], mix2[j][3]}));
            st16_nt(dst + 4, __builtin_bit_cast(u32x4, f32x4{mix2[j][4], mix2[j][5], mix2[j][6], mix2[j][7]}));
          }
        }
        if (tid == 0 && !flagw)
          st8_nt(f.ah.scal + 2 * (size_t)t, __builtin_bit_cast(u32x2, f32x2{pre2.anchor, pre2.total}));
      } else {
        pre[k] = token_pre<NT, NCH>(a, t, w, mix, lds_pre);
      }
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = tid + j * NT;
        pm2[k][j] = chunk_mix2(mix[j]);
        if (kOne) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            mix1[kOne ? j : 0][i] = mix[j][i];
            mg1[kOne ? j : 0][i] = mix[j][i] * gg[j][i];
          }
        } else if (c < CH) {
#pragma unroll
          for (int i = 0; i < 8; ++i) mixk[kOne ? 0 : k][kOne ? 0 : j][i] = mix[j][i];
        }
      }
      lds_barrier();  // lds_pre is reused by the next token
    }
  }

  // post: collect every token's new prefix from the mailbox. Each chunk's
  // post partials (and, for one token, new*gains) are formed as soon as it
  // arrives (its mix^2 partial already in pre); once the last chunk is in,
  // the mailbox words are re-armed and only the reduction and the output
  // remain.
  if (flagw) return;  // nothing stored yet (the look-ahead stores above skip it too)
  int tok[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) tok[k] = k < ntok ? o + k * NO : o;
  const __amdgpu_buffer_rsrc_t mbox =
      __builtin_amdgcn_make_buffer_rsrc(f.mailbox, 0, M * a.H * 2, kBufferDword3);
  // With two tokens per owner the post phase runs twice, as one copy of its
  // code: a dry pass right after pre() (the owners' idle time while W
  // streams), whose reductions run on zeros and whose stores go to empty
  // buffer ranges (the hardware drops them), then the real pass, which then
  // runs warm (64 tokens, K = 8192: 30.7 -> 30.3 us). With one token the
  // owner has no such slack (one token, K = 1024: +1.0 us; eight tokens,
  // K = 4096: +0.3 us), so it runs the real pass only.
  constexpr bool kDry = KT > 1;
  auto post = [&](const bool live) {
    const unsigned row_bytes = live ? (unsigned)(2 * a.H) : 0u;  // 0: stores dropped
    u32x4 nbits[KT][NCH];
    float pc[KT][NCH][4];
    float ngo[KT][NCH][8];  // new*gains, formed as each chunk arrives
    unsigned pending = 0, todo = 0;
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        nbits[k][j] = u32x4{0u, 0u, 0u, 0u};
        pc[k][j][0] = pc[k][j][1] = pc[k][j][2] = 0.0f;
        pc[k][j][3] = pm2[k][j];
        if (k < ntok && tid + j * NT < CH) pending |= 1u << (k * NCH + j);
      }
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) ngo[k][j][i] = 0.0f;
    if (!live) {  // every chunk "arrived" as zeros
      todo = pending;
      pending = 0;
    }
    // a chunk that has arrived: form its partials (stores wait until the end:
    // a wavefront's loads of the next round would wait for them too)
    auto absorb = [&](unsigned& bits) {
#pragma unroll
      for (int k = 0; k < KT; ++k)
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const unsigned bit = 1u << (k * NCH + j);
          if (bits & bit) {
            const int c = tid + j * NT;
            float nw[8], mx[8];
            unpack8(nbits[k][j], nw);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              mx[i] = kOne ? mix1[kOne ? j : 0][i] : mixk[kOne ? 0 : k][kOne ? 0 : j][i];
              ngo[k][j][i] = nw[i] * gg[j][i];
            }
            float q[3];
            chunk_post_new(nw, w[j], mx, q);
            pc[k][j][0] = q[0];
            pc[k][j][1] = q[1];
            pc[k][j][2] = q[2];
          }
        }
      bits = 0;
    };
    for (int spin = 0; pending != 0; ++spin) {
      u32x4 r[KT][NCH];
#pragma unroll
      for (int k = 0; k < KT; ++k)
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const bool p = pending & (1u << (k * NCH + j));
          const unsigned off = (unsigned)tok[k] * (unsigned)(2 * a.H) + 16u * (unsigned)(tid + j * NT);
          r[k][j] = __builtin_amdgcn_raw_buffer_load_b128(mbox, p ? off : kBufferOff, 0, kCacheSC1);
        }
      absorb(todo);  // the previous round's arrivals, while these loads are in flight
#pragma unroll
      for (int k = 0; k < KT; ++k)
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const unsigned bit = 1u << (k * NCH + j);
          const u32x4 v = r[k][j];
          if ((pending & bit) && v.x != kMailboxSentinel && v.y != kMailboxSentinel &&
              v.z != kMailboxSentinel && v.w != kMailboxSentinel) {
            pending &= ~bit;
            todo |= bit;
            nbits[k][j] = v;
          }
        }
      if (pending == 0) break;
      if (spin >= kSpinLimit) {  // gave up: flag the workspace (results invalid)
        __hip_atomic_store(&f.ws->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);  // 1: 0.02-0.04 us faster per step than 2 (0: same as 2, 8: 0.1 us slower)
    }
    absorb(todo);
    // re-arm the collected mailbox words for the next call (device scope, like
    // every mailbox access), one 16-byte store per chunk (two 8-byte stores
    // were 0.18 us slower per step at 8 tokens); nothing below waits for them
    const __amdgpu_buffer_rsrc_t rearm =
        __builtin_amdgcn_make_buffer_rsrc(f.mailbox, 0, live ? M * a.H * 2 : 0, kBufferDword3);
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = tid + j * NT;
        if (k < ntok && c < CH) {
          const u32x4 sent = {kMailboxSentinel, kMailboxSentinel, kMailboxSentinel, kMailboxSentinel};
          __builtin_amdgcn_raw_buffer_store_b128(sent, rearm, (unsigned)tok[k] * (unsigned)(2 * a.H) + 16u * (unsigned)c, 0, kCacheSC1);
        }
      }
    float pp[4 * KT];
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s4 = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) s4 += pc[k][j][i];  // chunk order, as post_partials
        pp[4 * k + i] = s4;
      }
    wg_sum<4 * KT, NW>(pp, lds_pre);  // lds_pre is free: pre() and the last pass end with a barrier
    // two tokens: both output coefficients first, so their scalar chains
    // overlap (64 tokens: 0.05-0.1 us per step; with one token the same order
    // was slower)
    OutCoefs sc[KT];
    if constexpr (kDry) {
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const float tot[4] = {pp[4 * k], pp[4 * k + 1], pp[4 * k + 2], pp[4 * k + 3]};
        sc[k] = out_coefs(a, pre[k], tot);
      }
    }

#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if (k < ntok) {
        const int t = o + k * NO;
        float nw[NCH][8], ng[NCH][8], mix[NCH][8], mg[NCH][8];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const int c = tid + j * NT;
          unpack8(nbits[k][j], nw[j]);
          if (kOne) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              mix[j][i] = mix1[kOne ? j : 0][i];
              mg[j][i] = mg1[kOne ? j : 0][i];
              ng[j][i] = ngo[k][j][i];
            }
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) mix[j][i] = mixk[kOne ? 0 : k][kOne ? 0 : j][i];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              ng[j][i] = ngo[k][j][i];
              mg[j][i] = mix[j][i] * gg[j][i];
            }
          }
        }
        if (a.write >= 0 && a.write < a.nb) {  // a scored slot: written after pre() read it
          uint16_t* row = a.blocks + t * a.bst_t + a.write * a.bst_b;
          if constexpr (kDry) {
            const __amdgpu_buffer_rsrc_t brow = __builtin_amdgcn_make_buffer_rsrc(row, 0, row_bytes, kBufferDword3);
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
              const int c = tid + j * NT;
              __builtin_amdgcn_raw_buffer_store_b128(nbits[k][j], brow, c < CH ? 16u * c : kBufferOff,
                                                     0, WT ? kCacheSC1 : kCacheNTStore);
            }
          } else {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
              const int c = tid + j * NT;
              if (c < CH) st16<WT>(row + (size_t)c * 8, nbits[k][j]);
            }
          }
        }
        const float tot[4] = {pp[4 * k], pp[4 * k + 1], pp[4 * k + 2], pp[4 * k + 3]};
        if constexpr (kDry) {
          float res[NCH][8];
          out_values<NT, NCH>(a, sc[k], nw, ng, mix, mg, gg, lds_fin, res);
          const __amdgpu_buffer_rsrc_t orow =
              __builtin_amdgcn_make_buffer_rsrc(a.out + (size_t)t * a.ld_out, 0, row_bytes, kBufferDword3);
#pragma unroll
          for (int j = 0; j < NCH; ++j) {
            const int c = tid + j * NT;
            __builtin_amdgcn_raw_buffer_store_b128(pack8(res[j]), orow, c < CH ? 16u * c : kBufferOff,
                                                   0, kCacheNTStore);
          }
        } else {
          finish_out<NT, NCH, false>(a, t, out_coefs(a, pre[k], tot), nw, ng, mix, mg, gg, lds_fin);
        }
        if (a.final_b) lds_barrier();  // lds_fin is reused by the next token
      }
    }
  };
  if constexpr (kDry) {
    const int passes = 2 + (__builtin_amdgcn_readfirstlane(M) >> 30);  // 2, opaque: one copy
#pragma clang loop unroll(disable)
    for (int pass = 0; pass < passes; ++pass) {
      post(pass + 1 == passes);
      lds_barrier();  // lds_pre is reused by the next pass
    }
  } else {
    post(true);
  }
}

// Four kernel templates over one body (rather than one kernel template with
// look-ahead and W-layout flags): hipcc emitted the host launch stub of only
// one of two kernel instantiations that differed in nothing but such a flag.
template <int RT, int TT, bool SPLIT>
__global__ __launch_bounds__(kTokenThreads) void fused_kernel(FusedParams f, int R, int G, int NO) {
  fused_body<RT, TT, SPLIT, false, false>(f, R, G, NO);
}

template <int RT, int TT, bool SPLIT>
__global__ __launch_bounds__(kTokenThreads) void fused_ahead_kernel(FusedParams f, int R, int G,
                                                                     int NO) {
  fused_body<RT, TT, SPLIT, true, false>(f, R, G, NO);
}

// W in the prepared layout (attnres_oproj_packed_run), without and with the
// look-ahead statistics (attnres_oproj_packed_ahead_run)
template <int RT, int TT, bool SPLIT>
__global__ __launch_bounds__(kTokenThreads) void fused_packed_kernel(FusedParams f, int R, int G,
                                                                      int NO) {
  fused_body<RT, TT, SPLIT, false, true>(f, R, G, NO);
}

template <int RT, int TT, bool SPLIT>
__global__ __launch_bounds__(kTokenThreads) void fused_packed_ahead_kernel(FusedParams f, int R,
                                                                            int G, int NO) {
  fused_body<RT, TT, SPLIT, true, true>(f, R, G, NO);
}

__global__ void workspace_init_kernel(unsigned* ws, size_t words) {
  const size_t header = kWorkspaceHeader / 4;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    ws[i] = i < header ? 0u : kMailboxSentinel;
}

hipError_t launch_workspace_init(void* ws, size_t bytes, hipStream_t stream) {
  const size_t words = bytes / 4;
  const int blocks = (int)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024);
  hipLaunchKernelGGL(workspace_init_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     static_cast<unsigned*>(ws), words);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; 256 if unknown).
int compute_units() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

template <int RT, int TT, bool SPLIT = false>
hipError_t go(const FusedParams& p, int R, int G, int NO, hipStream_t stream) {
  if (p.wrows > 0 && p.ah.mix)
    hipLaunchKernelGGL((fused_packed_ahead_kernel<RT, TT, SPLIT>), dim3(G + NO),
                       dim3(kTokenThreads), 0, stream, p, R, G, NO);
  else if (p.wrows > 0)
    hipLaunchKernelGGL((fused_packed_kernel<RT, TT, SPLIT>), dim3(G + NO), dim3(kTokenThreads), 0,
                       stream, p, R, G, NO);
  else if (p.ah.mix)
    hipLaunchKernelGGL((fused_ahead_kernel<RT, TT, SPLIT>), dim3(G + NO), dim3(kTokenThreads), 0,
                       stream, p, R, G, NO);
  else
    hipLaunchKernelGGL((fused_kernel<RT, TT, SPLIT>), dim3(G + NO), dim3(kTokenThreads), 0, stream,
                       p, R, G, NO);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused(const FusedParams& p, hipStream_t stream) {
  const int H = p.a.H, M = p.a.T;
  // owners: one token each up to 32 tokens, then two tokens each
  const int per_owner = M <= 32 ? 1 : kMaxTokensPerOwner;
  const int NO = (M + per_owner - 1) / per_owner;
  const int tt = (M + 15) / 16;
  // beyond 32 tokens: split K (alternate 2048-element blocks) over pairs of
  // workgroups with 64-row groups, when both and the owners fit the compute
  // units
  if (tt >= 3 && split_partial_bytes(M, H) > 0) {
    const int ng = (H + kSplitRows - 1) / kSplitRows;
    if (2 * ng + NO <= compute_units() && p.K >= 256) {
      FusedParams q = p;
      q.ng = ng;
      return tt == 3 ? go<4, 3, true>(q, kSplitRows, 2 * ng, NO, stream)
                     : go<4, 4, true>(q, kSplitRows, 2 * ng, NO, stream);
    }
  }
  // GEMM rows per workgroup: even, at most 32, leaving NO compute units free.
  // On prepared W, 28 or 30 become 32: whole 16-row MFMA tiles and fewer
  // producers move the same bytes (7168 rows, 8 tokens: 224 workgroups of 32
  // rows instead of 239 of 30, 13.71 -> 13.64 us; a copy with the same ring
  // streams W as fast with 224 workgroups as with 239 or 256). Not on
  // row-major W: workgroups 32 rows apart start 256 KiB apart there, and
  // their concurrent chunk loads then fall on the same memory channels
  // (K = 4096: 14.2 -> 18.0 us).
  int room = compute_units() - NO;
  if (room < 1) room = 1;
  int R = (H + room - 1) / room;
  R = (R + 1) & ~1;
  if (R < 2) R = 2;
  if (R >= 28 && p.wrows > 0) R = 32;
  if (R > 32) R = 32;
  const int G = (H + R - 1) / R;
  if (R > 16) {
    switch (tt) {
      case 1: return go<2, 1>(p, R, G, NO, stream);
      case 2: return go<2, 2>(p, R, G, NO, stream);
      case 3: return go<2, 3>(p, R, G, NO, stream);
      default: return go<2, 4>(p, R, G, NO, stream);
    }
  }
  switch (tt) {
    case 1: return go<1, 1>(p, R, G, NO, stream);
    case 2: return go<1, 2>(p, R, G, NO, stream);
    case 3: return go<1, 3>(p, R, G, NO, stream);
    default: return go<1, 4>(p, R, G, NO, stream);
  }
}

}  // namespace attnres
