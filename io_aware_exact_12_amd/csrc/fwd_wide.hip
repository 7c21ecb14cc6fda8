// Exact attention forward for wide heads (d = 256), bf16 / fp16, on gfx950.
//
// The same computation as the main forward kernel: for each query row the
// scores against the visible keys, their softmax and the weighted sum of the
// value rows, with the row statistics kept on chip so that no N x N matrix
// reaches HBM ("Flash Attention: IO-Aware Exact Attention", sections "Online
// softmax" and "Loop order changes which data is reloaded"; "FlashAttention --
// the same attention, made memory-aware", sections 02 and 03).
//
// At d = 256 a 32-query wave needs 128 accumulator registers for O^T and 64
// for its resident Q^T operands, so the kernel runs one 4-wave workgroup per
// CU (one wave per SIMD, up to 512 registers a wave) and two K/V stages of
// 64-key tiles (2 x 64 KB of LDS).  Per wave: 32 resident queries in the lane
// column of 32x32x16 MFMAs; for each 32-key half of a tile
//   S^T = K Q^T           (A = K rows from LDS, B = Q^T resident)
//   P^T = exp2(c S^T - c m)  against a lazily raised reference m
//   O^T += V^T P^T        (A = V^T by LDS transpose reads, B = P^T from registers)
// The reference only moves when a block's maximum exceeds it by more than
// kLazy (in log2 units): probabilities stay below 2^kLazy and the rescale of
// the 128 accumulators is rare.  The result does not depend on the
// reference, which only cancels between numerator and denominator.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "fa_internal.hpp"
#include "mfma_common.hpp"
#include "tile_common.hpp"

namespace fa {
namespace {

using namespace mfma;
using namespace tiles;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;

template <int D> struct WideLds {
  static constexpr int kK = 0;
  static constexpr int kV = STile<D>::kBytes;
  static constexpr int kStage = 2 * STile<D>::kBytes;
  static constexpr int kBytes = 2 * kStage;
};

template <bool IsBf16, int D, bool Causal>
__global__ __launch_bounds__(kThr, 1) void fwd_wide_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int H, int BH, int n_qblocks, float c,
    uint32_t q_sign, Layout lq, Layout in, Layout out) {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using T = STile<D>;
  using Ld = WideLds<D>;
  constexpr int kKs = D / 16, kDB = D / 32;
  static_assert(Ld::kBytes <= 160 * 1024, "two K/V stages fit the LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Ld::kBytes];

  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (Causal) qb = n_qblocks - 1 - qb;  // heaviest first
  const int b = bh / H, h = bh - b * H;
  const int q0 = qb * kRes, qw0 = q0 + 32 * wave, my_q = qw0 + l32;

  vec8 qf[kKs];
  load_resident<IsBf16, D>(qf, Q + (b * lq.sb + h * lq.sh), N, my_q, lq.sn, g, q_sign);

  const int last_row = min(N, q0 + kRes) - 1;
  const int n_tiles = Causal ? last_row / kT + 1 : (N + kT - 1) / kT;
  const bool wave_live = qw0 < N;
  const int64_t head = b * in.sb + h * in.sh;
  const uint16_t* k_h = K + head;
  const uint16_t* v_h = V + head;
  uint32_t src[T::kPerWave];
  T::sources(wave, lane, (uint32_t)(2 * in.sn), src);
  const uint32_t lds0 = lds_u32(smem);
  auto issue = [&](int it, int st) {
    const uint32_t base = lds0 + (uint32_t)(st * Ld::kStage);
    copy_tile<D>(base + Ld::kK, k_h, N, it * kT, in.sn, wave, src);
    copy_tile<D>(base + Ld::kV, v_h, N, it * kT, in.sn, wave, src);
  };

  f32x16 acc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) acc[i] = f32x16{};
  float m = -INFINITY;  // reference: raw (sign-adjusted) score of this lane's query
  float l = 0.f;        // this lane half's share of the row sum, relative to m

  issue(0, 0);
  wait_copies();
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int st = it & 1;
    if (it + 1 < n_tiles) issue(it + 1, st ^ 1);
    const uint8_t* k_lds = smem + st * Ld::kStage + Ld::kK;
    const uint8_t* v_lds = smem + st * Ld::kStage + Ld::kV;
    if (wave_live) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int ks0 = it * kT + 32 * kh;
        if ((Causal && ks0 > qw0 + 31) || ks0 >= N) continue;
        // register rr of lane half g holds key ks0 + 16 (rr >> 3) + 8 g + (rr & 7)
        f32x16 s = f32x16{};
        const int r = 32 * kh + l32;
#pragma unroll
        for (int kk = 0; kk < kKs; ++kk) s = E::mfma(row_frag<IsBf16, D>(k_lds, r, g, kk), qf[kk], s);
        if ((Causal && ks0 + 31 > qw0) || ks0 + 32 > N) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int kj = ks0 + 16 * (rr >> 3) + 8 * g + (rr & 7);
            if (kj >= N || (Causal && kj > my_q)) s[rr] = -INFINITY;
          }
        }
        float mx = s[0];
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
        mx = xhalf_max(mx);
        // (-inf) - (-inf) is NaN and compares false: a row that has seen no key
        // yet keeps its reference until a block shows it one
        if (__builtin_amdgcn_ballot_w64((mx - m) * c > kLazy) != 0) {
          const float m_new = fmaxf(m, mx);
          const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
          l *= alpha;
#pragma unroll
          for (int db = 0; db < kDB; ++db) acc[db] *= alpha;
          m = m_new;
        }
        const float neg_mc = m == -INFINITY ? 0.f : -m * c;
        u32x4 pw[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e], c, neg_mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e + 1], c, neg_mc));
          pw[e >> 2][e & 3] = E::pack2(p0, p1);
          l += p0 + p1;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            acc[db] = E::mfma(tr_frag<IsBf16, D>(v_lds, lane, 2 * kh + t, db),
                              __builtin_bit_cast(vec8, pw[t]), acc[db]);
      }
    }
    wait_copies();
    __syncthreads();
  }
  if (!wave_live) return;
  const float l_tot = xhalf_sum(l);
  if (my_q >= N) return;
  store_row<IsBf16, D>(O + (b * out.sb + h * out.sh), my_q, out.sn, g, acc, 1.0f / l_tot);
  if (LSE != nullptr && g == 0)
    LSE[(int64_t)bh * N + my_q] = ((m == -INFINITY ? 0.f : m * c) + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <bool IsBf16, int D, bool Causal>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int N = (int)a.N;
  const int BH = (int)(a.B * a.H);
  const int n_qblocks = (N + kRes - 1) / kRes;
  // c = |scale| * log2(e); a zero scale is run as the limit scale -> 0+ (every
  // exp2 argument rounds to 0, so visible keys weigh exactly 1)
  const float c = a.scale != 0.f ? __builtin_fabsf(a.scale) * 1.4426950408889634f : 1e-30f;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_wide_kernel<IsBf16, D, Causal>), dim3((unsigned)(n_qblocks * BH)), dim3(kThr),
                     0, stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, N, (int)a.H,
                     BH, n_qblocks, c, q_sign, a.lq, a.in, a.out);
  return hipGetLastError();
}

template <bool IsBf16>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
  return a.causal ? launch<IsBf16, 256, true>(a, s) : launch<IsBf16, 256, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_wide_bf16(const FwdArgs& a, hipStream_t s) { return dispatch<true>(a, s); }
hipError_t launch_fwd_wide_f16(const FwdArgs& a, hipStream_t s) { return dispatch<false>(a, s); }

}  // namespace fa
