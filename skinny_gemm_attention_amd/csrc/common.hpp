// Device helpers for gfx950 (CDNA4, wave64): bfloat16 packing, exact
// residual rounding, 16-byte loads, and fixed-order wavefront / workgroup
// reductions built on DPP and LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxBlocks = 8;   // saved blocks per token
constexpr int kMaxH = 8192;     // widest AttnRes row
constexpr int kMaxM = 64;       // tokens per GEMM call
constexpr float kLog2e = 1.4426950408889634f;

// ---- bfloat16 <-> float ----------------------------------------------------

// Low / high bfloat16 of a packed pair, widened exactly.
__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
  f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
  f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

// Round two floats to bfloat16 (nearest even; v_cvt_pk_bf16_f32), packed with
// `a` in the low half.
__device__ __forceinline__ unsigned pack2(float a, float b) {
  f32x2 p = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(p, bf16x2));
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 r;
  r.x = pack2(f[0], f[1]);
  r.y = pack2(f[2], f[3]);
  r.z = pack2(f[4], f[5]);
  r.w = pack2(f[6], f[7]);
  return r;
}

// -0.0 halves of a bfloat16 pair become +0.0 (gemm.ws_gemm page, positive_zero).
__device__ __forceinline__ unsigned positive_zero(unsigned w) {
  if ((w & 0xFFFFu) == 0x8000u) w &= 0xFFFF0000u;
  if ((w >> 16) == 0x8000u) w &= 0x0000FFFFu;
  return w;
}

// a + b for bfloat16 a and b, as a float whose rounding to bfloat16 (nearest
// even) is the correctly rounded bfloat16 sum. One float addition suffices:
// float carries 24 significant bits, at least 2 * 8 + 2, and for addition of
// two 8-bit-precision values rounding first to 24 bits and then to 8 never
// differs from rounding once (the double-rounding bound for addition,
// Figueroa 1995).
__device__ __forceinline__ float add_bf16_exact(float a, float b) { return a + b; }

// Reciprocal RMS of a row from its sum of squares (attn_res.kernel page,
// helper rstd): rsqrt(sum_sq / H + eps), v_rsq_f32.
__device__ __forceinline__ float rstd(float sum_sq, float inv_h, float eps) {
  return __builtin_amdgcn_rsqf(__builtin_fmaf(sum_sq, inv_h, eps));
}

// e^x through v_exp_f32 (2^x).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ---- memory -----------------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Raw buffer loads: an offset at or past num_records reads zeros without a
// memory access, which makes loads that some lanes (or some calls) must skip
// branch-free.
constexpr unsigned kBufferOff = 0xFFFFFFF0u;  // past num_records: reads zeros
constexpr int kBufferDword3 = 0x00020000;     // raw buffer, 32-bit data format
constexpr int kCacheNTLoad = 2;               // buffer-load cache policy: non-temporal
constexpr int kCacheNTStore = 2;              // buffer-store cache policy: non-temporal
// Streamed-once data (the weight matrix): non-temporal hint.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Output stores. Every tensor a kernel writes is read by a later kernel, not
// by this one, so no output store keeps its line in the caches:
//   * st16_nt / st8_nt: non-temporal (streaming) 16- or 8-byte store;
//   * st4_wt / st8_wt / st16_wt: written through to memory (device scope: sc1
//     global stores, issued as relaxed agent-scope atomic stores of 4 or 8
//     bytes), which leaves no dirty line in the L2 caches for the release at
//     the end of the kernel to write back. A 256-workgroup kernel storing
//     1 MiB took 0.2 us longer per launch with plain or non-temporal stores,
//     0.02 us with written-through ones; but written-through stores drain
//     slower, so a kernel that stores tens of KiB per workgroup (attnres_run:
//     5.4 -> 12.1 us at 256 tokens) keeps the non-temporal ones.
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st8_nt(void* p, u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st4_wt(void* p, unsigned v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st8_wt(void* p, u32x2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     __builtin_bit_cast(unsigned long long, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st16_wt(void* p, u32x4 v) {
  st8_wt(p, u32x2{v.x, v.y});
  st8_wt(reinterpret_cast<char*>(p) + 8, u32x2{v.z, v.w});
}
// One of the two, chosen at compile time by the kernel.
template <bool WT>
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  if constexpr (WT) st16_wt(p, v);
  else st16_nt(p, v);
}
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Blocks until every memory operation this wavefront has issued is complete:
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone). A completed device-scope
// store is visible to device-scope loads from any compute unit.
__device__ __forceinline__ void wait_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// vmcnt(N) lgkmcnt(0): this wavefront's memory operations except the N most
// recent have completed, and its LDS operations too.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);  // vmcnt(N) lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// vmcnt(n) lgkmcnt(0) for a wave-uniform 0 <= n <= N (waitcnt immediates
// exist only at compile time, hence the chain).
template <int N>
__device__ __forceinline__ void wait_vmem_upto(int n) {
  if constexpr (N == 0) {
    wait_vmem_n<0>();
  } else {
    if (n >= N) wait_vmem_n<N>();
    else wait_vmem_upto<N - 1>(n);
  }
}

// Workgroup barrier without a memory fence (the waits above are explicit).
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier for LDS traffic: waits for this wavefront's LDS operations
// (lgkmcnt(0)) but not for its global stores, which __syncthreads() would
// also drain (vmcnt(0)). Call from uniform control flow.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt and expcnt: no wait; lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- fixed-order reductions --------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// DPP move with a row mask: rows outside `ROW_MASK` read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes of a wavefront, in a fixed tree, left in lane 63:
// butterflies inside each 16-lane row (xor 1, xor 2, half-row mirror, row
// mirror; the two addends of every pair are the same numbers, so all lanes of
// a row agree bit for bit), then row_bcast:15 (row 1 += row 0, row 3 += row 2)
// and row_bcast:31 (row 3 += lane 31): lane 63 holds
// (row0 + row1) + (row2 + row3). Must be called with all lanes active.
__device__ __forceinline__ float wave_sum63(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  v += dpp_rows<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_rows<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// The same sum, returned to every lane.
__device__ __forceinline__ float wave_sum(float v) { return readlane(wave_sum63(v), 63); }

// The value of lane (l ^ X) (wave64), all VALU: X = 1, 2 are DPP quad
// permutations; X = 4, 8 take row_shl / row_shr by X (whichever points at the
// partner); X = 16, 32 use gfx950's v_permlane16_swap / v_permlane32_swap,
// which exchange rows 0 <-> 1 and 2 <-> 3 / lane halves.
template <int X>
__device__ __forceinline__ float xor_lane(float v) {
  const int lane = threadIdx.x & 63;
  if constexpr (X == 1) {
    return dpp<0xB1>(v);
  } else if constexpr (X == 2) {
    return dpp<0x4E>(v);
  } else if constexpr (X == 4 || X == 8) {
    const float up = dpp<0x100 + X>(v);    // row_shl: lane i reads lane i + X
    const float down = dpp<0x110 + X>(v);  // row_shr: lane i reads lane i - X
    return (lane & X) ? down : up;
  } else if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(X == 32, "xor partner");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// Sums K = 2^n values over the 64 lanes of a wavefront with about 2K lane
// exchanges instead of 6K: at level L < n each lane keeps half of its values
// (the half selected by lane bit L) and adds its partner's (lane ^ 2^L) copy
// of that half; the levels n..5 add the single remaining value across the
// partner. Every addition pairs a lane with a partner that computes the same
// sum with the operands swapped, so all lanes holding a value agree bit for
// bit. On return v[0] of lane l holds the total of value index
// k(l) = sum_L bit_L(l) * (K >> (L + 1)), i.e. the bit reverse of l mod K.
template <int K, int L = 0>
__device__ __forceinline__ void wave_multi_sum(float (&v)[K]) {
  if constexpr (L < 6) {
    const int lane = threadIdx.x & 63;
    constexpr int n = K >> L;  // values still held per lane (power of two, >= 1)
    if constexpr (n > 1) {
      const bool hi = (lane >> L) & 1;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float keep = hi ? v[n / 2 + i] : v[i];
        const float send = hi ? v[i] : v[n / 2 + i];
        v[i] = keep + xor_lane<(1 << L)>(send);
      }
    } else {
      v[0] += xor_lane<(1 << L)>(v[0]);
    }
    wave_multi_sum<K, L + 1>(v);
  }
}

// LDS floats wg_sum<K, NW> needs: the wavefront totals, then the K totals.
template <int K, int NW>
constexpr int wg_sum_lds = NW * K + K;

// Sums K per-thread partials over a workgroup of NW wavefronts: wavefront sums
// (wave_sum63 for K <= 4, wave_multi_sum beyond), then the NW wavefront
// totals in wavefront order (for K > 4 formed once by K threads and read
// back by every thread). Every thread gets the totals in v. `lds` holds wg_sum_lds<K, NW>
// floats and must not be reused by another reduction of the same workgroup
// until all threads have returned. Contains workgroup barriers: call from
// uniform control flow.
template <int K, int NW>
__device__ __forceinline__ void wg_sum(float (&v)[K], float* lds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if constexpr (K <= 4) {
    float t[K];
#pragma unroll
    for (int k = 0; k < K; ++k) t[k] = wave_sum63(v[k]);
    if (lane == 63) {
#pragma unroll
      for (int k = 0; k < K; ++k) lds[wave * K + k] = t[k];
    }
  } else {
    static_assert((K & (K - 1)) == 0 && K <= 64, "a power of two");
    float t[K];
#pragma unroll
    for (int k = 0; k < K; ++k) t[k] = v[k];
    wave_multi_sum<K>(t);
    if (lane < K) {
      int k = 0;  // bit reverse of lane within log2(K) bits
#pragma unroll
      for (int b = 0; (1 << b) < K; ++b) k |= ((lane >> b) & 1) * (K >> (b + 1));
      lds[wave * K + k] = t[0];
    }
  }
  lds_barrier();
  if constexpr (K <= 4) {  // few values: every thread adds the wavefront totals
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float s = lds[k];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += lds[w * K + k];
      v[k] = s;
    }
  } else {  // K threads add them once, every thread reads the K totals
    if ((int)threadIdx.x < K) {
      const int k = threadIdx.x;
      float s = lds[k];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += lds[w * K + k];
      lds[NW * K + k] = s;
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = lds[NW * K + k];
  }
}

}  // namespace attnres
