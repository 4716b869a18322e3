// Weight-stationary skinny GEMM core on the MFMA units of gfx950.
//
// The operation is WsGemm's y[M, N] = x[M, K] W[N, K]^T (vLLM gemm.ws_gemm
// page, module summary) for M <= 64 tokens: BF16 operands, FP32 accumulation,
// partial sums added in a fixed K order. A workgroup owns R consecutive rows
// of W; W and x reach the MFMA units through LDS (see GemmLds below).
//
// MFMA v_mfma_f32_16x16x32_bf16: A = 16 rows of W x 32 k, B = 32 k x 16
// tokens; lane l supplies row / token (l % 16) and k = 8 (l / 16) .. + 7. The
// accumulator of lane l holds D[4 (l / 16) + r][l % 16], r < 4: rows
// n0 + 4 (l / 16) + r of token (l % 16) of the tile.
#pragma once

#include "common.hpp"

namespace attnres {

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- LDS-staged core ---------------------------------------------------------
//
// W and x are staged through LDS by direct global->LDS
// loads (global_load_lds_dwordx4: lane l's 16 bytes land at M0 + 16 l, no
// VGPR involved), so the bytes a compute unit keeps in flight are bounded by
// LDS, not by registers, and every load instruction reads whole row segments
// (KCB contiguous bytes per row) instead of 64-byte MFMA fragments.
//
//   * K is cut into chunks of KE = KCB / 2 elements. A chunk holds, for the
//     workgroup's R rows of W and the M rows of x, KCB bytes per row; a ring
//     of NSLOT chunk slots keeps NSLOT - 1 chunks in flight while one is
//     consumed. All NW wavefronts load parts of every chunk (one instruction
//     per 1 KiB: 1024 / KCB rows) and consume it. With at least NW k-steps per
//     chunk, wavefront w takes the k-steps [w SPW, (w + 1) SPW) of each chunk
//     for all row tiles; with fewer (STEPS < NW), wavefront w takes k-step
//     w % STEPS for the row tiles of row group w / STEPS. Either way a
//     wavefront's partial sums run in K order, and the NP partials of an
//     output element are added in k-slice order.
//   * The core streams chunks of a K range [k_begin, k_begin + K) of each row:
//     blocks of cblock consecutive chunks, every cstride-th block, so two
//     workgroups can split K by taking alternate blocks (the caller adds
//     their partial products). cstride = cblock = 1 streams the whole range.
//   * Inside a row the 16-byte pieces are stored XOR-swizzled: piece p of a
//     row sits at position p ^ key, with key = (LDS row) & 15, or for the W
//     rows of a prepared W (global row) & 15. An MFMA fragment read (16
//     consecutive rows, one piece each) then touches 16 distinct bank groups.
//   * W is read either row-major (row n at W + n ldw) or from the tile-major
//     prepared layout (pack_kernel): planes of 128 k-values of every row,
//     each row's 256-byte segment already swizzled by its global row & 15, so
//     a load instruction reads whole contiguous 256-byte segments of
//     consecutive rows and lands in LDS in the order the reads expect; the
//     workgroups of a launch together sweep each plane front to back.
//   * Rows past R, tokens past M and pieces past K are never loaded. Stale LDS
//     in rows past R or tokens past M only reaches output rows / tokens that
//     are discarded (MFMA output elements are independent); k-steps that
//     straddle K are masked to zero in registers.
//   * One workgroup barrier per chunk: after it, chunk c is complete (each
//     wavefront waited for its own loads of c) and every wavefront has
//     finished reading chunk c - 1, whose slot is refilled next.
// Cache-policy operand of global_load_lds: the non-temporal bit.
constexpr int kCacheNT = 2;

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <int RT, int TT, int KCB, int NSLOT, bool PACKED = false>
struct GemmLds {
  static constexpr int NW = 8, NT = NW * 64;
  static constexpr int kQuads = RT * TT * 64;
  static constexpr int WROWS = RT * 16, ROWS = WROWS + TT * 16;
  static constexpr int SLOT = ROWS * KCB;
  static constexpr int kLdsBytes = NSLOT * SLOT;
  static constexpr int KE = KCB / 2;                 // k per chunk
  static constexpr int STEPS = KE / 32;              // 32-wide k-steps per chunk
  static constexpr int NP = STEPS < NW ? STEPS : NW; // k-partials per output element
  static constexpr int RH = NW / NP;                 // row groups across wavefronts
  static constexpr int SPW = STEPS / NP;             // k-steps per wavefront per chunk
  static constexpr int RTW = RT / RH;                // row tiles per wavefront
  static constexpr int PIECES = KCB / 16;            // 16-byte pieces per row segment
  static constexpr int RPI = 1024 / KCB;             // rows per load instruction
  static constexpr int MAXSEG = ((WROWS + TT * 16) / RPI + NW - 1) / NW;
  static_assert(NW % NP == 0 && STEPS % NP == 0 && RT % RH == 0, "wavefront split");
  static_assert(PIECES >= 16 && KCB <= 1024, "swizzle needs at least 16 pieces per row");
  static_assert(NSLOT >= 2, "ring");
  static_assert(NP * kQuads * 16 <= kLdsBytes, "the partials fit the ring");

  lds_char* ring;           // kLdsBytes of LDS
  const char* gp[MAXSEG];   // this lane's source for chunk 0 of each of its segments
  uint32_t dst[MAXSEG];     // segment offset inside a slot (wave-uniform)
  uint32_t kb[MAXSEG];      // byte offset of this lane's piece inside a chunk
  bool rv[MAXSEG];          // this lane's row exists
  uint32_t wstep;           // prepared W: bytes from one chunk of a row to the next
  int nseg, nwseg, nC, rot, K, cs, cbk, wave, kp, rh, r16, kq, akey;
  f32x4 acc[RTW][TT];

  // Chunks are consumed in the order rot, rot + 1, ..., wrapping around.
  __device__ __forceinline__ int phys(int c) const {
    const int p = c + rot;
    return p >= nC ? p - nC : p;
  }
  // Offset (in chunks, from k_begin) of this workgroup's p-th chunk: blocks
  // of cbk consecutive chunks, every cs-th block.
  __device__ __forceinline__ int coff(int p) const { return (p / cbk) * cbk * cs + p % cbk; }

  __device__ __forceinline__ void issue(int c) {
    const uint32_t ci = (uint32_t)coff(phys(c));
    const uint32_t cb = ci * KCB;                  // x (and row-major W): bytes into the row
    const uint32_t cw = PACKED ? ci * wstep : cb;  // W: bytes to this chunk
    lds_char* slot = ring + (c % NSLOT) * SLOT;
    if (KCB < 1024 && cb + KCB <= (uint32_t)(2 * K)) {
      // a whole chunk: every lane loads (lanes of rows past R or M read row
      // 0 again, into LDS rows whose outputs are discarded). Measured faster
      // with 256- and 512-byte segments, slower with 1 KiB ones.
#pragma unroll
      for (int i = 0; i < MAXSEG; ++i) {
        if (i < nwseg)  // W is read once: non-temporal
          __builtin_amdgcn_global_load_lds(gp[i] + cw, slot + dst[i], 16, 0, kCacheNT);
        else if (i < nseg)
          __builtin_amdgcn_global_load_lds(gp[i] + cb, slot + dst[i], 16, 0, 0);
      }
      return;
    }
    // a chunk that K cuts: lanes past K skip their load (a prepared W is
    // zero-padded, so all its lanes load: kb = 0)
#pragma unroll
    for (int i = 0; i < MAXSEG; ++i) {
      if (i < nseg) {
        if (rv[i] && cb + kb[i] < (uint32_t)(2 * K)) {
          if (i < nwseg)  // W is read once: non-temporal
            __builtin_amdgcn_global_load_lds(gp[i] + cw, slot + dst[i], 16, 0, kCacheNT);
          else
            __builtin_amdgcn_global_load_lds(gp[i] + cb, slot + dst[i], 16, 0, 0);
        }
      }
    }
  }


  // Sets up this wavefront's segments for the k range [k_begin, k_begin + K_)
  // of rows [row0, row0 + rows) (blocks of cblock chunks, every cstride-th
  // block) and issues the first NSLOT - 1 chunks. With rot_ > 0 the chunks
  // are taken in rotated order (workgroups that share x then read different
  // parts of it at a time); the order is fixed per call. W is row-major with
  // row stride ldw, or with PACKED the prepared layout of a matrix of wrows
  // rows (ldw unused; k_begin a multiple of 128; fewer than 2^32 bytes).
  __device__ __forceinline__ void start(const uint16_t* __restrict__ x, int64_t ldx,
                                        const uint16_t* __restrict__ W, int64_t ldw, int M,
                                        int k_begin, int K_, int row0, int rows, char* lds,
                                        int rot_ = 0, int cstride = 1, int cblock = 1,
                                        int wrows = 0) {
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    kp = wave % NP;
    rh = wave / NP;
    r16 = lane & 15;
    kq = lane >> 4;
    K = K_;
    cs = cstride;
    cbk = cblock;
    ring = (lds_char*)lds;
    {
      const int nt = K > 0 ? (K + KE - 1) / KE : 0;  // chunks of the range
      const int per = cbk * cs;
      nC = (nt / per) * cbk + min(cbk, nt % per);
    }
    rot = nC > 0 ? rot_ % nC : 0;
    const int wseg = (rows + RPI - 1) / RPI, xseg = (M + RPI - 1) / RPI;
    const int S = wseg + xseg;
    nseg = wave < S ? (S - wave + NW - 1) / NW : 0;
    nwseg = wave < wseg ? (wseg - wave + NW - 1) / NW : 0;  // W segments come first
    const int lr = lane / PIECES, q = lane % PIECES;
    // swizzle key of the W rows this lane reads as A: the global row for a
    // prepared W (swizzled when it was prepared), else the LDS row
    if (PACKED) {
      akey = (row0 + r16) & 15;
      wstep = (uint32_t)(KCB / 256) * (uint32_t)wrows * 256u;
    }
#pragma unroll
    for (int i = 0; i < MAXSEG; ++i) {
      const int sidx = wave + i * NW;
      const bool isw = sidx < wseg;
      const int r = (isw ? sidx : sidx - wseg) * RPI + lr;  // row within W rows or x rows
      rv[i] = isw ? r < rows : r < M;
      const int rr = rv[i] ? r : 0;
      if (PACKED && isw) {
        // prepared W: position q of this row's chunk is position q % 16 of
        // its segment in plane k_begin / 128 + q / 16 (already swizzled)
        gp[i] = reinterpret_cast<const char*>(W) +
                ((size_t)(k_begin / 128 + q / 16) * wrows + (size_t)(row0 + rr)) * 256 + 16 * (q % 16);
        kb[i] = 0;
      } else {
        const int p = q ^ (r & 15);  // LDS row & 15 (W rows start at LDS row 0, x rows at WROWS)
        gp[i] = isw ? reinterpret_cast<const char*>(W + (size_t)(row0 + rr) * ldw + k_begin) + 16 * p
                    : reinterpret_cast<const char*>(x + (size_t)rr * ldx + k_begin) + 16 * p;
        kb[i] = 16 * p;
      }
      dst[i] = __builtin_amdgcn_readfirstlane(((isw ? 0 : WROWS) + (sidx < wseg ? sidx : sidx - wseg) * RPI) * KCB);
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < NSLOT - 1 && c < nC; ++c) issue(c);
  }

  // One chunk's operands for this wavefront: the A (W rows) and B (x rows)
  // fragments of its k-steps. live: the k-step starts inside K (wave-uniform);
  // cut: this lane's 8 k-values lie past K, so its operands count as zero.
  struct Frags {
    u32x4 a[SPW][RTW], b[SPW][TT];
    bool live[SPW], cut[SPW];
  };

  // Issues the LDS reads of chunk c's fragments; nothing waits for them here.
  __device__ __forceinline__ void load_frags(int c, Frags& f) const {
    const lds_char* slot = ring + (c % NSLOT) * SLOT;
    const int cbase = coff(phys(c)) * KE;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int ks = kp * SPW + j;
      const int k0 = cbase + ks * 32;
      f.live[j] = k0 < K;
      f.cut[j] = k0 + 8 * kq >= K;
      if (f.live[j]) {
        const int offb = 16 * ((ks * 4 + kq) ^ r16);
        const int offa = PACKED ? 16 * ((ks * 4 + kq) ^ akey) : offb;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
          f.a[j][rt] = *reinterpret_cast<const lds_u32x4*>(slot + ((rh * RTW + rt) * 16 + r16) * KCB + offa);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          f.b[j][tt] = *reinterpret_cast<const lds_u32x4*>(slot + (WROWS + tt * 16 + r16) * KCB + offb);
      }
    }
  }

  // The matrix-core products of one chunk's fragments, in k-step order.
  __device__ __forceinline__ void mma(Frags& f) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      if (f.live[j]) {
        if (f.cut[j]) {
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) f.a[j][rt] = zero;
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) f.b[j][tt] = zero;
        }
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = mfma_bf16(f.a[j][rt], f.b[j][tt], acc[rt][tt]);
      }
    }
  }

  // Waits until chunk c is in LDS for every wavefront (and every wavefront has
  // finished reading chunk c - 1, whose slot is refilled here), issues chunk
  // c + NSLOT - 1 and the LDS reads of chunk c's fragments.
  __device__ __forceinline__ void step(int c, Frags& f) {
    const int ahead = min(c + NSLOT - 2, nC - 1) - c;  // chunks after c already issued
    wait_vmem_upto<MAXSEG * (NSLOT - 2)>(nseg * ahead);  // also lgkmcnt(0): earlier fragment reads
    wg_barrier();
    if (c + NSLOT - 1 < nC) issue(c + NSLOT - 1);
    load_frags(c, f);
  }

  // Reads chunk c's fragments and runs their products at once (wide tiles).
  __device__ __forceinline__ void compute(int c) {
    const lds_char* slot = ring + (c % NSLOT) * SLOT;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int ks = kp * SPW + j;
      const int k0 = coff(phys(c)) * KE + ks * 32;
      if (k0 < K) {
        const int offb = 16 * ((ks * 4 + kq) ^ r16);
        const int offa = PACKED ? 16 * ((ks * 4 + kq) ^ akey) : offb;
        u32x4 a[RTW], b[TT];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
          a[rt] = *reinterpret_cast<const lds_u32x4*>(slot + ((rh * RTW + rt) * 16 + r16) * KCB + offa);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          b[tt] = *reinterpret_cast<const lds_u32x4*>(slot + (WROWS + tt * 16 + r16) * KCB + offb);
        if (k0 + 32 > K && k0 + 8 * kq >= K) {
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) a[rt] = zero;
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) b[tt] = zero;
        }
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = mfma_bf16(a[rt], b[tt], acc[rt][tt]);
      }
    }
  }

  // Consumes every chunk; returns with all loads complete and all wavefronts
  // past their last LDS read of the ring. With two row tiles and up to two
  // token tiles the loop is software-pipelined by one chunk: the products of
  // chunk c - 1 run while chunk c's fragment reads are in flight (two
  // fragment sets in turn; the products keep chunk order). Other tiles read
  // and multiply each chunk in turn: written as load_frags + mma, that loop
  // made the compiler wait for the chunk's own LDS traffic before its
  // fragment reads at four token tiles (64 tokens, K = 8192: 31.0 -> 36.8 us),
  // and the 16-row tile of 1 KiB segments ran 0.4 us slower pipelined
  // (8 tokens, K = 7168, N = 4096).
  __device__ __forceinline__ void finish() {
    if (TT > 2 || RT == 1) {
      for (int c = 0; c < nC; ++c) {
        const int ahead = min(c + NSLOT - 2, nC - 1) - c;  // chunks after c already issued
        wait_vmem_upto<MAXSEG * (NSLOT - 2)>(nseg * ahead);
        wg_barrier();
        if (c + NSLOT - 1 < nC) issue(c + NSLOT - 1);
        compute(c);
      }
    } else if (nC > 0) {
      Frags f0, f1;
      step(0, f0);
      int c = 1;
      for (; c + 1 < nC; c += 2) {
        step(c, f1);
        mma(f0);
        step(c + 1, f0);
        mma(f1);
      }
      if (c < nC) {
        step(c, f1);
        mma(f0);
        mma(f1);
      } else {
        mma(f0);
      }
    }
    wait_vmem_n<0>();
    wg_barrier();
  }

  // This wavefront's partial tiles: red[(kp * kQuads) + quad].
  __device__ __forceinline__ void stash(f32x4* red) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        red[((kp * RT + rh * RTW + rt) * TT + tt) * 64 + lane] = acc[rt][tt];
  }

  // Sum over the k-partials, in k-slice order, of quad q < kQuads. All NP
  // reads are issued before the first addition (one LDS round trip).
  __device__ static __forceinline__ f32x4 gather(const f32x4* red, int q) {
    f32x4 p[NP];
#pragma unroll
    for (int w = 0; w < NP; ++w) p[w] = red[w * kQuads + q];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s = p[0];
#pragma unroll
    for (int w = 1; w < NP; ++w) s += p[w];
    return s;
  }

  // Token and first row (relative to row0) of quad q.
  __device__ static __forceinline__ void quad_coords(int q, int& m, int& r) {
    const int rt = q / (TT * 64), tt = (q / 64) % TT, ln = q & 63;
    m = tt * 16 + (ln & 15);
    r = rt * 16 + 4 * (ln >> 4);
  }
};

// Chunk shape per tile shape (measured on MI355X): 512-byte row segments in
// four slots for two row tiles and one token tile; 1 KiB segments in four
// slots (128 KB) for a single row tile (wsgemm_run at M <= 16, N = 4096: 5%
// faster than three slots; five do not fit beside the fused kernel's other
// LDS); 512-byte segments beyond 16 tokens, where x dominates a chunk.
template <int RT, int TT, bool PACKED = false>
using GemmLdsFor = GemmLds<RT, TT, (TT == 1 && RT == 1 ? 1024 : 512),
                           (TT == 1 ? 4 : TT == 2 ? 4 : 3), PACKED>;

// Split-K tiles for more than 32 tokens: 64 rows (four row tiles) per
// workgroup over half of K, 256-byte row segments in four slots; wavefronts
// split into four k-steps by two row groups.
constexpr int kSplitRows = 64;
template <int TT, bool PACKED = false>
using GemmLdsSplit = GemmLds<4, TT, 256, (TT <= 4 ? 4 : 3), PACKED>;  // three slots beyond 64 tokens

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
// Written through (WT) or non-temporal (a later kernel reads them).
template <bool WT>
__device__ __forceinline__ void store_quad_pairs(uint16_t* row, int r, int rows, u32x2 v) {
  if constexpr (WT) {
    if (r < rows) st4_wt(row + r, v.x);
    if (r + 2 < rows) st4_wt(row + r + 2, v.y);
  } else {
    if (r < rows) __builtin_nontemporal_store(v.x, reinterpret_cast<unsigned*>(row + r));
    if (r + 2 < rows) __builtin_nontemporal_store(v.y, reinterpret_cast<unsigned*>(row + r + 2));
  }
}

}  // namespace attnres
