// Exact attention forward for bf16 / fp16 on gfx950 (MI355X), using MFMA.
//
// What is computed: for every query row, O = softmax(scale * q K^T) V over the
// visible keys and LSE = ln sum exp(scale * q . k), with the N x N scores never
// leaving the chip.  Query blocks are the outer loop and stay resident in
// registers; key/value tiles are the inner loop and stream through LDS
// ("Flash Attention: IO-Aware Exact Attention", section "Loop order changes
// which data is reloaded").  Each query row carries a running maximum m, a
// denominator l and an unnormalised d-wide numerator a; a tile that raises the
// maximum rescales both l and a by alpha = exp(m_old - m_new), and O = a / l is
// formed once at the end (same page, section "Online softmax makes tiling
// exact", and the FlashAttention-2 remark there about the unnormalised
// accumulator).
//
// Mapping to CDNA4:
//  * One workgroup = 4 waves = 128 query rows (32 rows per wave).  The grid is
//    (query block, head, batch) work items, heaviest causal blocks first.
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 MFMA: the
//    K tile is the A operand (read from LDS), Q^T the B operand (held in
//    registers for the whole loop).  The accumulator then holds one query per
//    lane column, so the row statistics live in that lane: lanes l and l+32
//    share a query and split its keys, and a single cross-half exchange per
//    tile gives the row maximum.
//  * K rows are written to LDS in a permuted order chosen so that, in the S^T
//    accumulator, lane half g holds 8 *consecutive* keys per 8 registers.  The
//    probabilities, rounded to the input type, are then directly the B operand
//    of O^T += V^T P^T, with no LDS round trip; V is stored transposed in LDS so
//    its A operand is one 16-byte read.  O^T keeps the query in the lane column
//    too, so alpha and 1/l are per-lane scalars.
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA per score.
//  * K/V tiles are double-buffered in LDS with the next tile prefetched into
//    registers while the current one is consumed; one barrier per tile.
//  * Causal: tiles entirely above a wave's rows are skipped, the mask is only
//    evaluated on tiles that cross the diagonal or the sequence end.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <cstdint>

#include "fa_internal.hpp"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <bool IsBf16> struct Elt;
template <> struct Elt<true> {
  using scalar = __bf16;
  using vec8 = bf16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Elt<false> {
  using scalar = _Float16;
  using vec8 = f16x8;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Row of the LDS K tile that holds key `key` (0..63) of the tile.  Within each
// 32-key half, MFMA output row 8b + 4g + j must carry key
// 16*(b>>1) + 8g + 4*(b&1) + j so that accumulator registers r = 0..7 of lane
// half g hold keys 8g..8g+7 and r = 8..15 hold keys 16+8g..16+8g+7.
__device__ __forceinline__ int k_lds_row(int key) {
  const int half = key & 32;
  const int kk = key & 31;
  const int j = kk & 3, t = (kk >> 2) & 1, g = (kk >> 3) & 1, bh = (kk >> 4) & 1;
  const int b = 2 * bh + t;
  return half + 8 * b + 4 * g + j;
}

template <int D>
struct Smem {
  static constexpr int kStrideK = D + 8;     // elements; +16 B per row against bank conflicts
  static constexpr int kStrideV = kBN + 8;   // V^T rows are keys-contiguous
  static constexpr int kKElems = kBN * kStrideK;
  static constexpr int kVElems = D * kStrideV;
  static constexpr int kStageElems = kKElems + kVElems;
  static constexpr int kBytes = 2 * kStageElems * 2;
};

template <bool IsBf16, int D, bool Causal>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int BH, int n_qblocks, float c,
    uint32_t q_sign) {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using S = Smem<D>;
  constexpr int kKs = D / 16;          // MFMA k-steps for S^T = K Q^T
  constexpr int kDB = D / 32;          // 32-row blocks of O^T
  constexpr int kChunks = D / 8;       // 16-byte chunks per row
  constexpr int kKLoads = kBN * kChunks / kThreads;  // K chunks per thread per tile
  constexpr int kVKeys = kBN * kChunks / kThreads;   // V rows per thread per tile (same count)
  static_assert(kKLoads * kThreads == kBN * kChunks, "K tile must split evenly");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * S::kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // work item: heaviest causal query blocks first
  const int bid = blockIdx.x;
  const int bh = bid % BH;
  int qb = bid / BH;
  if (Causal) qb = n_qblocks - 1 - qb;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;

  const int q0_blk = qb * kBM;
  const int q0 = q0_blk + 32 * wave;           // first row of this wave
  const int my_q = q0 + l32;                   // this lane's query row
  const int last_blk_row = min(N, q0_blk + kBM) - 1;
  const int n_tiles = Causal ? (last_blk_row / kBN + 1) : (N + kBN - 1) / kBN;
  const int wave_last_row = min(N, q0 + 32) - 1;  // < q0 when the wave is past N
  const bool wave_active = q0 < N;

  // ---- Q^T fragments (B operand): lane holds query my_q, d = 16*ks + 8*g + 0..7
  vec8 qf[kKs];
  {
    const bool ok = my_q < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(Qh + (int64_t)(ok ? my_q : 0) * D);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      u32x4 raw = ok ? src[2 * ks + g] : u32x4{0, 0, 0, 0};
      raw ^= q_sign;  // negative scale: flip the sign of q, exactly
      qf[ks] = __builtin_bit_cast(vec8, raw);
    }
  }

  // ---- tile loaders: global -> registers -> LDS
  u32x4 kreg[kKLoads];
  u32x4 vreg[kVKeys];
  // V: thread owns d-chunk vc and keys vk0 .. vk0 + kVKeys - 1
  const int vc = tid % kChunks;
  const int vk0 = (tid / kChunks) * kVKeys;

  auto load_tile = [&](int j) {
    const int key0 = j * kBN;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int cidx = tid + i * kThreads;
      const int key = key0 + cidx / kChunks;
      const int ch = cidx % kChunks;
      kreg[i] = key < N ? *reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D + ch * 8)
                        : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kVKeys; ++i) {
      const int key = key0 + vk0 + i;
      vreg[i] = key < N ? *reinterpret_cast<const u32x4*>(Vh + (int64_t)key * D + vc * 8)
                        : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* ks = smem + stage * S::kStageElems;
    uint16_t* vt = ks + S::kKElems;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int cidx = tid + i * kThreads;
      const int key = cidx / kChunks;
      const int ch = cidx % kChunks;
      *reinterpret_cast<u32x4*>(ks + k_lds_row(key) * S::kStrideK + ch * 8) = kreg[i];
    }
    // transpose V: element e of chunk vc of key vk0+i goes to Vt[vc*8+e][vk0+i]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t vals[kVKeys];
#pragma unroll
      for (int i = 0; i < kVKeys; ++i) {
        const uint32_t w = vreg[i][e >> 1];
        vals[i] = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffff);
      }
      uint16_t* dst = vt + (vc * 8 + e) * S::kStrideV + vk0;
      if constexpr (kVKeys == 4) {
        u32x2 pk = {(uint32_t)vals[0] | ((uint32_t)vals[1] << 16),
                    (uint32_t)vals[2] | ((uint32_t)vals[3] << 16)};
        *reinterpret_cast<u32x2*>(dst) = pk;
      } else {
        static_assert(kVKeys == 2, "V transpose handles 2 or 4 keys per thread");
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)vals[0] | ((uint32_t)vals[1] << 16);
      }
    }
  };

  // ---- running row state (per lane: query my_q, keys of lane half g)
  f32x16 acc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of raw scores q.k (sign-adjusted)
  float l_part = 0.f;       // this lane half's share of the denominator

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int stage = j & 1;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) load_tile(j + 1);

    const int key0 = j * kBN;
    const bool wave_needs = wave_active && (!Causal || key0 <= wave_last_row);
    if (wave_needs) {
      const uint16_t* ks = smem + stage * S::kStageElems;
      const uint16_t* vt = ks + S::kKElems;

      // S^T = K Q^T for keys 0-31 and 32-63 of the tile
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* krow = ks + (kb * 32 + l32) * S::kStrideK + 8 * g;
#pragma unroll
        for (int kk = 0; kk < kKs; ++kk) {
          const vec8 a = *reinterpret_cast<const vec8*>(krow + 16 * kk);
          s[kb] = E::mfma(a, qf[kk], s[kb]);
        }
      }

      // masks: keys above the diagonal (causal) and keys past the end
      const bool need_mask = (Causal && key0 + kBN - 1 > q0) || (key0 + kBN > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
            const bool hide = key >= N || (Causal && key > my_q);
            s[kb][r] = hide ? -INFINITY : s[kb][r];
          }
      }

      // row maximum: in-lane over 32 keys, then across the two lane halves
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      // every processed tile holds a visible key for every valid row (key 0 is
      // always visible and tile 0 comes first), so m_new is finite for valid rows
      const float m_scaled = (m_new == -INFINITY) ? 0.f : m_new * c;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run * c - m_scaled);
      m_run = m_new;

      // p = exp2(c*s - c*m_new); masked entries give exactly 0
      float rowsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_scaled));
          if (need_mask) p = (s[kb][r] == -INFINITY) ? 0.f : p;
          s[kb][r] = p;
          rowsum += p;
        }
      l_part = alpha * l_part + rowsum;

      // P^T operands: step t covers keys 16t..16t+15; lane half g holds 8 of them
      vec8 pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = s[t >> 1][8 * (t & 1) + e];
        pb[t] = __builtin_convertvector(pf, vec8);
      }

      // O^T = alpha * O^T + V^T P^T
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        acc[db] *= alpha;
        const uint16_t* vrow = vt + (db * 32 + l32) * S::kStrideV + 8 * g;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const vec8 a = *reinterpret_cast<const vec8*>(vrow + 16 * t);
          acc[db] = E::mfma(a, pb[t], acc[db]);
        }
      }
    }

    if (has_next) store_tile(stage ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;

  // ---- epilogue: O = a / l once, LSE = ln(sum) of the scaled scores
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / l_tot;
  if (my_q < N) {
    uint16_t* orow = O + head_off + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        typedef __attribute__((ext_vector_type(4))) float f32x4;
        f32x4 v4 = {acc[db][4 * grp] * inv, acc[db][4 * grp + 1] * inv,
                    acc[db][4 * grp + 2] * inv, acc[db][4 * grp + 3] * inv};
        typedef __attribute__((ext_vector_type(4))) typename E::scalar h4_t;
        const auto h4 = __builtin_convertvector(v4, h4_t);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * grp + 4 * g) = __builtin_bit_cast(u32x2, h4);
      }
    if (LSE != nullptr && g == 0) {
      LSE[(int64_t)bh * N + my_q] = (m_run * c + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

template <bool IsBf16, int D, bool Causal>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int N = (int)a.N;
  const int BH = (int)(a.B * a.H);
  const int n_qblocks = (N + kBM - 1) / kBM;
  const dim3 grid((unsigned)(n_qblocks * BH));
  const float c = __builtin_fabsf(a.scale) * kLog2e;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<IsBf16, D, Causal>), grid, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, N, BH,
                     n_qblocks, c, q_sign);
  return hipGetLastError();
}

template <bool IsBf16>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
  if (a.d == 128) return a.causal ? launch<IsBf16, 128, true>(a, s) : launch<IsBf16, 128, false>(a, s);
  return a.causal ? launch<IsBf16, 64, true>(a, s) : launch<IsBf16, 64, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) { return dispatch<true>(a, s); }
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t s) { return dispatch<false>(a, s); }

}  // namespace fa
