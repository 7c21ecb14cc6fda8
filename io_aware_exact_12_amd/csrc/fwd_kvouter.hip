// Forward pass in the original key/value-outer loop order, kept beside the
// query-outer kernel as the comparison the pages draw between the two orders
// ("Flash Attention: IO-Aware Exact Attention", section "Loop order changes
// which data is reloaded"; "FlashAttention -- the same attention, made
// memory-aware", sections 03 and 04).
//
// One workgroup owns one (batch, head).  Its outer loop walks the key/value
// tiles: each tile is copied into LDS once.  The inner loop walks every query
// tile that can see the key tile; for each, every wave
//   - reloads its 32 query rows and their row state (normalised output O,
//     running maximum m and denominator l, all fp32) from device memory,
//   - forms the scores of the 64 keys by MFMA, their maximum and exp2 weights,
//   - merges them into the state: m' = max(m, m_t),
//     l' = e^(m - m') l + e^(m_t - m') l_t,
//     O' = (e^(m - m') l O + e^(m_t - m') P V) / l'   (section 03's update),
//   - writes the state back.
// After the last key tile the same lanes turn the state into O in the input
// dtype and the natural-log LSE.  The state round trip per (key tile, query
// tile) pair is the traffic the query-outer order avoids; this kernel exists to
// measure it, not to be fast.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "fa_internal.hpp"
#include "mfma_common.hpp"

namespace fa {
namespace {

using namespace mfma;

constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvBM = 32 * kKvWaves;  // query rows per query tile
constexpr int kKvBN = 64;             // keys per key/value tile

// LDS of one key/value tile.  K row `row` holds key k_row_key(row) of the tile
// (the order that leaves score registers 0..7 of lane half g on keys
// 8g..8g+7), V rows are in key order; paddings as in the query-outer kernel.
template <int D> struct KvLds {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kKStride = kRowBytes + 16;
  static constexpr int kVStride = kRowBytes + 64;
  static constexpr int kKBytes = kKvBN * kKStride;
  static constexpr int kBytes = kKBytes + kKvBN * kVStride;
};

template <bool IsBf16, int D, bool Causal>
__global__ __launch_bounds__(kKvThreads, 1) void fwd_kv_outer_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ o_ws,
    float* __restrict__ m_ws, float* __restrict__ l_ws, int N, float c, uint32_t q_sign) {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using L = KvLds<D>;
  constexpr int kKs = D / 16;       // score MFMAs per 32 keys
  constexpr int kDB = D / 32;       // 32-row blocks of O^T
  constexpr int kChunks = D / 8;    // 16-byte chunks per row
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::kBytes];
  uint8_t* const k_lds = smem;
  uint8_t* const v_lds = smem + L::kKBytes;

  const int bh = blockIdx.x;
  const int64_t head_off = (int64_t)bh * N * D;
  const int64_t row_off = (int64_t)bh * N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int n_kt = (N + kKvBN - 1) / kKvBN;
  const int n_qt = (N + kKvBM - 1) / kKvBM;
  const uint32_t head_bytes = (uint32_t)N * L::kRowBytes;
  const __amdgpu_buffer_rsrc_t q_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Q + head_off), 0, (int)head_bytes, kRsrcFlags);
  // score A operand: LDS row l32 of a 32-key half, 16-byte chunk 2 kk + g
  const int k_base = l32 * L::kKStride + g * 16;
  // V^T A operand by transpose reads (the query-outer kernel's pattern)
  const int grp = lane >> 4, s16 = lane & 15;
  const int v_base = (8 * g + (s16 >> 2)) * L::kVStride + 2 * (16 * (grp & 1) + 4 * (s16 & 3));

  for (int jt = 0; jt < n_kt; ++jt) {
    const int key0 = jt * kKvBN;
    __syncthreads();  // every wave is done with the previous tile
    for (int ci = tid; ci < kKvBN * kChunks; ci += kKvThreads) {
      const int row = ci / kChunks, col = ci % kChunks;
      const int kk = key0 + k_row_key(row), vk = key0 + row;
      u32x4 kv = u32x4{}, vv = u32x4{};
      if (kk < N) kv = *reinterpret_cast<const u32x4*>(K + head_off + (int64_t)kk * D + col * 8);
      if (vk < N) vv = *reinterpret_cast<const u32x4*>(V + head_off + (int64_t)vk * D + col * 8);
      *reinterpret_cast<u32x4*>(k_lds + row * L::kKStride + col * 16) = kv;
      *reinterpret_cast<u32x4*>(v_lds + row * L::kVStride + col * 16) = vv;
    }
    __syncthreads();

    // causal: query tiles before the one holding row key0 see none of these keys
    const int it_first = Causal ? key0 / kKvBM : 0;
    for (int it = it_first; it < n_qt; ++it) {
      const int q0 = it * kKvBM + 32 * wave;
      if (q0 >= N || (Causal && q0 + 31 < key0)) continue;  // wave-uniform
      const int my_q = q0 + l32;
      const bool row_ok = my_q < N;

      // query fragments, reloaded for every key tile (rows past N read as 0)
      vec8 qf[kKs];
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        u32x4 raw = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rs, my_q * L::kRowBytes + (2 * ks + g) * 16, 0, 0));
        raw ^= q_sign;  // negative scale: flip the sign of q, exactly
        qf[ks] = __builtin_bit_cast(vec8, raw);
      }

      // scores of the two 32-key halves, masked; register r of lane half g
      // holds key key0 + 32 h + 16 (r >> 3) + 8 g + (r & 7)
      f32x16 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[h] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < kKs; ++kk)
          s[h] = E::mfma(*reinterpret_cast<const vec8*>(k_lds + h * 32 * L::kKStride + k_base + kk * 32),
                         qf[kk], s[h]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * h + 16 * (r >> 3) + 8 * g + (r & 7);
          if (key >= N || (Causal && key > my_q)) s[h][r] = -INFINITY;
        }
      }
      float mt = s[0][0];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[h][r]);
      mt = xhalf_max(mt);  // the tile's row maximum (raw score units)
      const float mt_off = mt == -INFINITY ? 0.f : -mt * c;

      // tile weights p = exp2(c (s - m_t)), their fp32 row sum, and P^T packed
      // as the B operand of the PV MFMAs
      u32x4 pw[2][2];
      float lt = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][2 * e], c, mt_off));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][2 * e + 1], c, mt_off));
          pw[h][e >> 2][e & 3] = E::pack2(p0, p1);
          lt += p0 + p1;
        }
      lt = xhalf_sum(lt);

      // P V for the tile: O^T d = 32 db + 8 (r/4) + 4 g + r%4 of query my_q
      f32x16 pv[kDB];
#pragma unroll
      for (int db = 0; db < kDB; ++db) pv[db] = f32x16{};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int f = 0; f < 2 * kDB; ++f) {
          const int db = f >> 1, tt = f & 1;
          const uint8_t* vp = v_lds + v_base + (32 * h + 16 * tt) * L::kVStride + 64 * db;
          const auto lo = E::read_tr((const lds_void*)vp);
          const auto hi = E::read_tr((const lds_void*)(vp + 4 * L::kVStride));
          pv[db] = E::mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                           __builtin_bit_cast(vec8, pw[h][tt]), pv[db]);
        }

      // row state before this key tile (none before the first)
      float m_prev = -INFINITY, l_prev = 0.f;
      float* const orow = o_ws + (head_off + (int64_t)my_q * D);
      f32x16 ost[kDB];
#pragma unroll
      for (int db = 0; db < kDB; ++db) ost[db] = f32x16{};
      if (jt > 0 && row_ok) {
        m_prev = m_ws[row_off + my_q];
        l_prev = l_ws[row_off + my_q];
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(orow + 32 * db + 8 * gq + 4 * g);
#pragma unroll
            for (int x = 0; x < 4; ++x) ost[db][4 * gq + x] = v4[x];
          }
      }

      // merge (section 03's update, with exp2 and the scale folded into c)
      const float m_new = fmaxf(m_prev, mt);
      const float a_prev = m_prev == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_prev - m_new) * c);
      const float a_tile = mt == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mt - m_new) * c);
      const float l_new = a_prev * l_prev + a_tile * lt;
      const float inv = l_new > 0.f ? 1.0f / l_new : 0.f;  // no visible key yet: state stays empty
      const float w_old = l_prev * a_prev * inv, w_new = a_tile * inv;
      if (row_ok) {
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            f32x4 v4;
#pragma unroll
            for (int x = 0; x < 4; ++x)
              v4[x] = __builtin_fmaf(ost[db][4 * gq + x], w_old, pv[db][4 * gq + x] * w_new);
            *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * gq + 4 * g) = v4;
          }
        // both lane halves hold the same m and l and write them, so that every
        // lane reads back its own store
        m_ws[row_off + my_q] = m_new;
        l_ws[row_off + my_q] = l_new;
      }
    }
  }

  // O in the input dtype and LSE = ln(l) + m * scale, read back by the lanes
  // that wrote the state
  typedef __attribute__((ext_vector_type(4))) typename E::scalar h4_t;
  for (int it = 0; it < n_qt; ++it) {
    const int my_q = it * kKvBM + 32 * wave + l32;
    if (my_q >= N) continue;
    const float* orow = o_ws + (head_off + (int64_t)my_q * D);
    uint16_t* out = O + head_off + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * g;
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(orow + d0);
        *reinterpret_cast<u32x2*>(out + d0) = __builtin_bit_cast(u32x2, __builtin_convertvector(v4, h4_t));
      }
    if (LSE != nullptr && g == 0) {
      const float m = m_ws[row_off + my_q], l = l_ws[row_off + my_q];
      LSE[row_off + my_q] = (m * c + __builtin_amdgcn_logf(l)) * kLn2;
    }
  }
}

template <bool IsBf16, int D, bool Causal>
hipError_t launch(const FwdArgs& a, void* ws, hipStream_t stream) {
  const int N = (int)a.N;
  const int BH = (int)(a.B * a.H);
  const int64_t rows = (int64_t)BH * N;
  float* o_ws = static_cast<float*>(ws);
  float* m_ws = o_ws + rows * D;
  float* l_ws = m_ws + rows;
  // c = |scale| * log2(e), a zero scale run as the limit scale -> 0+ (the
  // query-outer kernel's convention); a negative scale flips q
  const float c = a.scale != 0.f ? __builtin_fabsf(a.scale) * 1.4426950408889634f : 1e-30f;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kv_outer_kernel<IsBf16, D, Causal>), dim3((unsigned)BH), dim3(kKvThreads), 0,
                     stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, o_ws, m_ws,
                     l_ws, N, c, q_sign);
  return hipGetLastError();
}

template <bool IsBf16>
hipError_t dispatch(const FwdArgs& a, void* ws, hipStream_t s) {
  if (a.d == 128) return a.causal ? launch<IsBf16, 128, true>(a, ws, s) : launch<IsBf16, 128, false>(a, ws, s);
  if (a.d == 96) return a.causal ? launch<IsBf16, 96, true>(a, ws, s) : launch<IsBf16, 96, false>(a, ws, s);
  return a.causal ? launch<IsBf16, 64, true>(a, ws, s) : launch<IsBf16, 64, false>(a, ws, s);
}

}  // namespace

size_t kv_outer_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return (size_t)(B * H * N) * (size_t)(4 * d + 8);
}
hipError_t launch_fwd_kv_outer_bf16(const FwdArgs& a, void* ws, hipStream_t s) {
  return dispatch<true>(a, ws, s);
}
hipError_t launch_fwd_kv_outer_f16(const FwdArgs& a, void* ws, hipStream_t s) {
  return dispatch<false>(a, ws, s);
}

}  // namespace fa
