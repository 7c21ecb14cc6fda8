// Streamed-tile helpers shared by the backward kernels and the wide-head
// forward: 64-row tiles copied HBM -> LDS with buffer_load ... lds in a
// permuted, XOR-swizzled row order, the MFMA operand reads on them, and the
// resident per-lane operands and row stores of a 4-wave workgroup that keeps
// 32 rows per wave in the lane column of 32x32x16 MFMAs.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "mfma_common.hpp"

namespace fa {
namespace tiles {

using namespace mfma;

constexpr int kW = 4;              // waves per workgroup
constexpr int kThr = 64 * kW;
constexpr int kRes = 32 * kW;      // resident rows (keys or queries) per workgroup
constexpr int kT = 64;             // streamed tile rows

// LDS row of logical index `idx` (0..63) of a streamed tile: MFMA output row
// 8b + 4g + j of each 32-row half holds index 16 (b >> 1) + 8 g + 4 (b & 1) + j,
// i.e. bits 2 and 3 of the index are swapped (the map is its own inverse).
__device__ __forceinline__ int tile_row(int idx) {
  const int half = idx & 32, kk = idx & 31;
  const int j = kk & 3, b1 = (kk >> 2) & 1, g = (kk >> 3) & 1, bh = (kk >> 4) & 1;
  return half + 16 * bh + 8 * b1 + 4 * g + j;
}

// A streamed tile of 64 rows of D elements, rows in the permuted order above,
// no padding.  The 16-byte chunks of LDS row r are XOR-swizzled by swz(r) so
// that both ways the tile is read are free of bank conflicts: 16 lanes reading
// one chunk of 16 consecutive rows (row operands), and 32 lanes reading 64
// contiguous bytes of 4 consecutive rows (transpose reads).
template <int D> struct STile {
  // LDS row pitch and the data of a row: d = 96 rows (12 chunks) sit in rows
  // of 16 chunks, so the 16-chunk swizzle of d = 128 applies; their last four
  // chunks are filled from past the row's data and never read.
  static constexpr int kDataBytes = 2 * D;
  static constexpr int kRowBytes = D == 96 ? 256 : 2 * D;
  static constexpr int kBytes = kT * kRowBytes;
  static constexpr int kCopies = kBytes / 1024;  // wave-wide 1 KB copies per tile
  static constexpr int kPerWave = kCopies / kW;
  static_assert(kPerWave * kW == kCopies, "tile copies split evenly over the waves");
  static __device__ __forceinline__ int swz(int r) {
    return D != 64 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  // byte offset in the tile of 16-byte chunk c of LDS row r
  static __device__ __forceinline__ int at(int r, int c) { return r * kRowBytes + 16 * (c ^ swz(r)); }
  // Tile-relative source offsets of this wave's copies (rows row_bytes apart
  // in device memory): copy i of wave w fills LDS bytes [(w + kW i) KB, +1 KB),
  // lane l the 16 bytes at 16 l.
  static __device__ __forceinline__ void sources(int wave, int lane, uint32_t row_bytes,
                                                 uint32_t (&src)[kPerWave]) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int byte = (wave + kW * i) * 1024 + 16 * lane;
      const int r = byte / kRowBytes, phys = (byte % kRowBytes) / 16;
      src[i] = (uint32_t)tile_row(r) * row_bytes + (uint32_t)(16 * (phys ^ swz(r)));
    }
  }
};

// HBM -> LDS copy of 4 bytes per lane: lane l writes LDS bytes
// [lds_addr + 4 l, +4) with the dword at byte offset voff of rsrc (zero past
// its size).  Same M0 handling as dma16.
__device__ __forceinline__ void dma4(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}

// Copy rows [row0, row0 + 64) of a [rows][D] view with row stride sn
// elements (zeros past `rows`) into the swizzled tile at LDS address
// lds_addr: this wave's share.  The buffer ends after the last row's data, so
// rows past `rows` (at least sn >= D elements further on) read as zero.
template <int D>
__device__ __forceinline__ void copy_tile(uint32_t lds_addr, const uint16_t* base, int rows, int row0,
                                          int64_t sn, int wave,
                                          const uint32_t (&src)[STile<D>::kPerWave]) {
  using T = STile<D>;
  const int left = rows - row0;
  const i32x4 rs = make_rsrc(base + (int64_t)row0 * sn,
                             left > 0 ? (uint32_t)(left - 1) * (uint32_t)(2 * sn) + (uint32_t)T::kDataBytes : 0u);
#pragma unroll
  for (int i = 0; i < T::kPerWave; ++i) dma16(rs, lds_addr + (uint32_t)((wave + kW * i) * 1024), src[i]);
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// Wait for all of this wave's HBM -> LDS copies.
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transpose-read A operand whose rows are the D dimension and whose 16-wide k
// dimension runs over 16 consecutive logical tile rows (k step t, d block db):
// lane s of each 16-lane group reads logical row 16 t + 8 g + 4 h + s/4
// (LDS row 16 t + 8 h + 4 g + s/4), columns 32 db + 16 (group & 1) + 4 (s & 3)
// .. + 3, for h = 0 (elements 0..3) and h = 1 (elements 4..7).
template <bool IsBf16, int D>
__device__ __forceinline__ typename Elt<IsBf16>::vec8 tr_frag(const uint8_t* tile, int lane, int t, int db) {
  using E = Elt<IsBf16>;
  using T = STile<D>;
  const int g = lane >> 5, grp = lane >> 4, s16 = lane & 15;
  const int col = 2 * (16 * (grp & 1) + 4 * (s16 & 3)) + 64 * db;  // byte column
  const int r0 = 16 * t + 4 * g + (s16 >> 2);
  const auto lo = E::read_tr((const lds_void*)(tile + T::at(r0, col >> 4) + (col & 15)));
  const auto hi = E::read_tr((const lds_void*)(tile + T::at(r0 + 8, col >> 4) + (col & 15)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row operand (A of a 32x32x16 MFMA) for k step kk: LDS row r, chunk 2 kk + g.
template <bool IsBf16, int D>
__device__ __forceinline__ typename Elt<IsBf16>::vec8 row_frag(const uint8_t* tile, int r, int g, int kk) {
  return *reinterpret_cast<const typename Elt<IsBf16>::vec8*>(tile + STile<D>::at(r, 2 * kk + g));
}

// Resident operand of one lane: row `row` of a [rows][D] view with row stride
// sn elements as the MFMA B operand (d = 16 ks + 8 g + 0..7), zero past
// `rows`, optionally sign-flipped.
template <bool IsBf16, int D>
__device__ __forceinline__ void load_resident(typename Elt<IsBf16>::vec8 (&f)[D / 16],
                                              const uint16_t* base, int rows, int row, int64_t sn,
                                              int g, uint32_t sign) {
  const uint32_t row_bytes = (uint32_t)(2 * sn);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)base, 0, (int)((uint32_t)(rows - 1) * row_bytes + 2 * D), kRsrcFlags);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 raw = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((uint32_t)row * row_bytes) + (2 * ks + g) * 16, 0, 0));
    raw ^= sign;
    f[ks] = __builtin_bit_cast(typename Elt<IsBf16>::vec8, raw);
  }
}

// Store one lane's column of a transposed accumulator (rows = d) as row `row`
// of a view with row stride sn elements, multiplied by `mul` and rounded to
// the element type.
template <bool IsBf16, int D, int NA>
__device__ __forceinline__ void store_row(uint16_t* base, int row, int64_t sn, int g,
                                          const f32x16 (&acc)[NA], float mul) {
  static_assert(NA >= D / 32, "one accumulator per 32 columns");
  using E = Elt<IsBf16>;
  typedef __attribute__((ext_vector_type(4))) typename E::scalar h4_t;
  uint16_t* orow = base + (int64_t)row * sn;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 v4 = {acc[db][4 * gq] * mul, acc[db][4 * gq + 1] * mul,
                        acc[db][4 * gq + 2] * mul, acc[db][4 * gq + 3] * mul};
      *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * gq + 4 * g) =
          __builtin_bit_cast(u32x2, __builtin_convertvector(v4, h4_t));
    }
}


}  // namespace tiles
}  // namespace fa
