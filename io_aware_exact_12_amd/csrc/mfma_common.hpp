// Device helpers shared by the gfx950 MFMA attention kernels (forward and
// backward): vector types, the 32x32x16 MFMA wrappers, LDS transpose reads,
// HBM -> LDS copies, buffer resources and cross-half lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>
#include <utility>

namespace fa {
namespace mfma {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLn2 = 0.6931471805599453f;
// buffer resource word 3 for raw (untyped) buffer access on CDNA
constexpr int kRsrcFlags = 0x00020000;

typedef __attribute__((ext_vector_type(4))) short i16x4;

// gfx950 LDS transpose read: within each 16-lane group, output lane i receives
// element (i & 3) of the 8-byte chunks addressed by lanes (i >> 2) + 4k,
// k = 0..3 (one element from each of four source lanes).
__device__ __forceinline__ i16x4 read_tr16(const lds_void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

typedef __attribute__((ext_vector_type(4))) int i32x4;

// HBM -> LDS copy of 16 bytes per lane: lane l writes LDS bytes
// [lds_addr + 16 l, +16) with the 16 bytes at byte offset voff of the buffer
// rsrc (zeros when voff is past the buffer's size).  Issued as inline assembly
// so the compiler does not treat every later LDS read as a possible alias of
// the copy (it would wait for all copies in flight); completion is tracked by
// the caller with explicit vmcnt waits before the workgroup barrier.  M0, which
// carries the LDS address, is saved and restored around the copy.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}

// Groups of such copies in one asm statement (M0 saved and restored once):
// copies 0.. use rsrc a (K), then b (V), the last one rsrc x.
__device__ __forceinline__ void dma_group5(const i32x4& a, const i32x4& b, const i32x4& x,
                                           uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3,
                                           uint32_t l4, uint32_t v0, uint32_t v1, uint32_t v2,
                                           uint32_t v3, uint32_t v4) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\tbuffer_load_dwordx4 %9, %1, 0 offen lds\n\t"
      "s_mov_b32 m0, %5\n\tbuffer_load_dwordx4 %10, %1, 0 offen lds\n\t"
      "s_mov_b32 m0, %6\n\tbuffer_load_dwordx4 %11, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %7\n\tbuffer_load_dwordx4 %12, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %8\n\tbuffer_load_dwordx4 %13, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(a), "s"(b), "s"(x), "s"(l0), "s"(l1), "s"(l2), "s"(l3), "s"(l4), "v"(v0), "v"(v1),
        "v"(v2), "v"(v3), "v"(v4)
      : "memory");
}
__device__ __forceinline__ void dma_group3(const i32x4& a, const i32x4& b, const i32x4& x,
                                           uint32_t l0, uint32_t l1, uint32_t l2, uint32_t v0,
                                           uint32_t v1, uint32_t v2) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\tbuffer_load_dwordx4 %7, %1, 0 offen lds\n\t"
      "s_mov_b32 m0, %5\n\tbuffer_load_dwordx4 %8, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %6\n\tbuffer_load_dwordx4 %9, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(a), "s"(b), "s"(x), "s"(l0), "s"(l1), "s"(l2), "v"(v0), "v"(v1), "v"(v2)
      : "memory");
}

// Four copies: two with rsrc a, one with b, the last with x (l0, l1 -> a).
__device__ __forceinline__ void dma_group4a(const i32x4& a, const i32x4& b, const i32x4& x,
                                            uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3,
                                            uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\tbuffer_load_dwordx4 %8, %1, 0 offen lds\n\t"
      "s_mov_b32 m0, %5\n\tbuffer_load_dwordx4 %9, %1, 0 offen lds\n\t"
      "s_mov_b32 m0, %6\n\tbuffer_load_dwordx4 %10, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %7\n\tbuffer_load_dwordx4 %11, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(a), "s"(b), "s"(x), "s"(l0), "s"(l1), "s"(l2), "s"(l3), "v"(v0), "v"(v1), "v"(v2), "v"(v3)
      : "memory");
}
// Four copies: one with rsrc a, two with b, the last with x (l1, l2 -> b).
__device__ __forceinline__ void dma_group4b(const i32x4& a, const i32x4& b, const i32x4& x,
                                            uint32_t l0, uint32_t l1, uint32_t l2, uint32_t l3,
                                            uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\tbuffer_load_dwordx4 %8, %1, 0 offen lds\n\t"
      "s_mov_b32 m0, %5\n\tbuffer_load_dwordx4 %9, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %6\n\tbuffer_load_dwordx4 %10, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %7\n\tbuffer_load_dwordx4 %11, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(a), "s"(b), "s"(x), "s"(l0), "s"(l1), "s"(l2), "s"(l3), "v"(v0), "v"(v1), "v"(v2), "v"(v3)
      : "memory");
}

// Buffer resource (base, size in bytes) for raw, bounds-checked access.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kRsrcFlags;
  return r;
}

template <bool V> struct BoolTag { static constexpr bool value = V; };

// f(std::integral_constant<int, 0>{}), .., f(std::integral_constant<int, N-1>{}):
// a loop whose index is a compile-time constant in every iteration, unrolled
// by construction (a long unrolled schedule must not fall back to a runtime
// loop with dynamically indexed register arrays).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <bool IsBf16> struct Elt;
template <> struct Elt<true> {
  using scalar = __bf16;
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 h2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
  }
  using vec8 = bf16x8;
  using vec4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 read_tr(const lds_void* p) {
    return __builtin_bit_cast(vec4, read_tr16(p));
  }
};
template <> struct Elt<false> {
  using scalar = _Float16;
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) _Float16 h2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
  }
  using vec8 = f16x8;
  using vec4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 read_tr(const lds_void* p) {
    return __builtin_bit_cast(vec4, read_tr16(p));
  }
};

// Key (0..63 within the tile) stored in K-tile LDS row `row`.  MFMA output row
// 8b + 4g + j of each 32-row half carries key 16*(b>>1) + 8g + 4*(b&1) + j, so
// that accumulator registers 0..7 of lane half g hold keys 8g..8g+7 and
// registers 8..15 hold keys 16+8g..16+8g+7.
__device__ __forceinline__ int k_row_key(int row) {
  const int half = row & 32, rr = row & 31;
  const int b = rr >> 3, g = (rr >> 2) & 1, j = rr & 3;
  return half + 16 * (b >> 1) + 8 * g + 4 * (b & 1) + j;
}

__device__ __forceinline__ float xhalf_max(float x) {
  // v_permlane32_swap with both operands x returns (x_lo | x_lo, x_hi | x_hi)
  // per lane half; their max is the max over lanes l and l ^ 32.
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
// The same over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (v_permlane16_swap
// pairs lanes l and l ^ 16).  Max and sum are commutative, so all four lanes
// get bitwise the same result.
__device__ __forceinline__ float quad_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return xhalf_max(fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])));
}
__device__ __forceinline__ float quad_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return xhalf_sum(__builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Kernel modes: plain (causal or not), causal sliding window, block-sparse.
constexpr int kModePlain = 0, kModeWindow = 1, kModeSparse = 2;
// Block-sparse masks have blocks of 64 x 64; a workgroup's list of tiles
// holds at most kMaxSparseTiles entries of 32 bits (tile index | bits << 16)
// plus 16 words of per-wave counts.
constexpr int kSparseBlock = 64;
constexpr int kMaxSparseTiles = 2048;
constexpr int kSparseBytes = 4 * kMaxSparseTiles + 64;

// Compact, in order, the items i in [0, n) whose bits_of(i) is nonzero into
// list[] as i | bits << 16 (bits < 2^16); every thread of the workgroup
// (kWaves waves) calls this, and its barriers.  counts: kWaves words of LDS
// after the list.  Returns the number of entries (wave-uniform).
template <int kWaves, typename F>
__device__ __forceinline__ int compact_tiles(uint32_t* list, int n, F bits_of) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t* counts = list + kMaxSparseTiles;
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += 64 * kWaves) {
    const int i = c0 + tid;
    const uint32_t bits = i < n ? bits_of(i) : 0u;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(bits != 0);
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) counts[wave] = (uint32_t)__builtin_popcountll(bal);
    __syncthreads();
    int off = base, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int cw = (int)counts[w];
      off += w < wave ? cw : 0;
      total += cw;
    }
    if (bits != 0) list[off + rank] = (uint32_t)i | (bits << 16);
    base += total;
    __syncthreads();  // counts are rewritten by the next chunk; the list is complete
  }
  return __builtin_amdgcn_readfirstlane(base);
}

}  // namespace mfma
}  // namespace fa
