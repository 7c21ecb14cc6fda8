// Tail rows of an unmasked bf16 / fp16 forward, with the keys split over the
// waves of a workgroup.
//
// The main forward kernel gives each workgroup 256 query rows.  When N is a
// little past a multiple of 256 (N = 4097, say) the last, nearly empty query
// block of every head still streams every key through one wave, a second
// round of workgroups as long as a full one.  Here one workgroup per head
// takes those rows (at most 32, one wave's worth) and splits the keys
// instead: wave w walks the 32-key blocks w, w + 8, .., each with its own
// running maximum, denominator and unnormalised numerator, in the same
// online-softmax recurrence ("Flash Attention: IO-Aware Exact Attention",
// section "Online softmax makes tiling exact").  The eight states are merged
// at the end with the same rescaling, alpha = exp(m_w - m), in wave order, so
// the result is deterministic.  O = a / l and LSE = m + ln l as in the main
// kernel.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "fa_internal.hpp"
#include "mfma_common.hpp"
#include "tile_common.hpp"

namespace fa {
namespace {

using namespace mfma;
using namespace tiles;

constexpr int kTW = 8;             // waves per workgroup
constexpr int kTB = 32;            // keys per block
constexpr int kTThr = 64 * kTW;

// A 32-key block in the streamed-tile format (the first half of STile<D>):
// rows in the permuted order, 16-byte chunks XOR-swizzled.
template <int D> struct TailBlock {
  using T = STile<D>;
  static constexpr int kBytes = kTB * T::kRowBytes;
  static constexpr int kChunks = kBytes / 1024;  // wave-wide 1 KB copies, all by one wave
  static_assert(kChunks * 1024 == kBytes, "whole 1 KB copies");
  // per-lane source offset of copy i (rows row_bytes apart in device memory)
  static __device__ __forceinline__ uint32_t source(int i, int lane, uint32_t row_bytes) {
    const int byte = i * 1024 + 16 * lane;
    const int r = byte / T::kRowBytes, phys = (byte % T::kRowBytes) / 16;
    return (uint32_t)tile_row(r) * row_bytes + (uint32_t)(16 * (phys ^ T::swz(r)));
  }
};

template <bool IsBf16, int D>
__global__ __launch_bounds__(kTThr, 1) void fwd_tail_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int r0, int H, float c, uint32_t q_sign,
    Layout lq, Layout in, Layout lv, Layout out) {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using TB = TailBlock<D>;
  constexpr int kKs = D / 16, kDB = D / 32;
  constexpr int kWaveBytes = 2 * TB::kBytes;       // this wave's K block, then its V block
  constexpr int kSumStride = 16 * kDB + 1;          // merge buffer: floats per lane
  static_assert(64 * kSumStride * 4 <= kTW * kWaveBytes, "the merge buffer fits in the blocks");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kTW * kWaveBytes];
  __shared__ float m_part[kTW][64];

  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int my_q = r0 + l32;

  vec8 qf[kKs];
  load_resident<IsBf16, D>(qf, Q + (b * lq.sb + h * lq.sh), N, my_q, lq.sn, g, q_sign);

  const uint16_t* k_h = K + (b * in.sb + h * in.sh);
  const uint16_t* v_h = V + (b * lv.sb + h * lv.sh);
  const uint32_t k_row = (uint32_t)(2 * in.sn), v_row = (uint32_t)(2 * lv.sn);
  uint32_t src_k[TB::kChunks], src_v[TB::kChunks];
#pragma unroll
  for (int i = 0; i < TB::kChunks; ++i) {
    src_k[i] = TB::source(i, lane, k_row);
    src_v[i] = TB::source(i, lane, v_row);
  }
  const uint8_t* kt = smem + wave * kWaveBytes;
  const uint8_t* vt = kt + TB::kBytes;
  const uint32_t kt_lds = lds_u32(kt), vt_lds = lds_u32(vt);

  f32x16 acc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) acc[i] = f32x16{};
  float m = -INFINITY;  // running maximum of the raw (sign-adjusted) scores of this lane's query
  float l = 0.f;        // this lane half's share of the denominator, relative to m
  const int n_blk = (N + kTB - 1) / kTB;

  // Copies of block u's K (or V) rows into this wave's buffer; rows past N
  // read as zeros.  The next block's K rows are copied once this block's score
  // MFMAs have read the K buffer, its V rows once the PV MFMAs have read the V
  // buffer, so each copy overlaps the rest of the block.
  auto issue = [&](int u, bool is_v) {
    const int row0 = u * kTB, left = N - row0;
    if (is_v) {
      const i32x4 rv = make_rsrc(v_h + (int64_t)row0 * lv.sn, (uint32_t)(left - 1) * v_row + 2 * D);
#pragma unroll
      for (int i = 0; i < TB::kChunks; ++i) dma16(rv, vt_lds + (uint32_t)(i * 1024), src_v[i]);
    } else {
      const i32x4 rk = make_rsrc(k_h + (int64_t)row0 * in.sn, (uint32_t)(left - 1) * k_row + 2 * D);
#pragma unroll
      for (int i = 0; i < TB::kChunks; ++i) dma16(rk, kt_lds + (uint32_t)(i * 1024), src_k[i]);
    }
  };
  if (wave < n_blk) {
    issue(wave, false);
    issue(wave, true);
  }
  for (int u = wave; u < n_blk; u += kTW) {
    const int left = N - u * kTB;
    const bool next = u + kTW < n_blk;
    wait_copies();

    // S^T = K Q^T; register rr of lane half g holds key row0 + 16 (rr >> 3) + 8 g + (rr & 7)
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk) s = E::mfma(row_frag<IsBf16, D>(kt, l32, g, kk), qf[kk], s);
    // the K operand reads have returned (each MFMA waited for its own)
    if (next) issue(u + kTW, false);
    if (left < kTB) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        if (16 * (rr >> 3) + 8 * g + (rr & 7) >= left) s[rr] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
    const float m_new = fmaxf(m, xhalf_max(mx));  // finite: the block holds a key < N
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < kDB; ++db) acc[db] *= alpha;
    const float neg_mc = -m * c;
    u32x4 pw[2];
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e], c, neg_mc));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e + 1], c, neg_mc));
      pw[e >> 2][e & 3] = E::pack2(p0, p1);
      sum += p0 + p1;
    }
    l += sum;
    // O^T += V^T P^T.  Every operand read returns before its MFMA issues, so
    // the next copy into the V buffer cannot overtake a read.
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        acc[db] = E::mfma(tr_frag<IsBf16, D>(vt, lane, t, db), __builtin_bit_cast(vec8, pw[t]), acc[db]);
    if (next) issue(u + kTW, true);
  }

  // Merge: m = max over the waves; each wave rescales its l and a by
  // alpha_w = exp(m_w - m) and the rescaled states are added in wave order in
  // LDS (the blocks are free: every wave is past the barrier).
  m_part[wave][lane] = m;
  __syncthreads();
  float m_all = -INFINITY;
#pragma unroll
  for (int w = 0; w < kTW; ++w) m_all = fmaxf(m_all, m_part[w][lane]);
  const float a_me = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - m_all) * c);
  float* sum = reinterpret_cast<float*>(smem) + lane * kSumStride;
  for (int w = 0; w < kTW; ++w) {
    if (w == wave) {
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float mine = a_me * acc[db][r];
          sum[16 * db + r] = w == 0 ? mine : sum[16 * db + r] + mine;
        }
      sum[16 * kDB] = w == 0 ? a_me * l : sum[16 * kDB] + a_me * l;
    }
    __syncthreads();
  }
  if (wave != 0) return;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = sum[16 * db + r];
  const float l_tot = xhalf_sum(sum[16 * kDB]);
  if (my_q >= N) return;
  store_row<IsBf16, D>(O + (b * out.sb + h * out.sh), my_q, out.sn, g, acc, 1.0f / l_tot);
  if (LSE != nullptr && g == 0)
    LSE[(int64_t)bh * N + my_q] = (m_all * c + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <bool IsBf16, int D>
hipError_t launch(const FwdArgs& a, int64_t r0, hipStream_t stream) {
  // c = |scale| * log2(e); a zero scale is run as the limit scale -> 0+
  const float c = a.scale != 0.f ? __builtin_fabsf(a.scale) * 1.4426950408889634f : 1e-30f;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_tail_kernel<IsBf16, D>), dim3((unsigned)(a.B * a.H)), dim3(kTThr), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, (int)a.N,
                     (int)r0, (int)a.H, c, q_sign, a.lq, a.in, a.lv, a.out);
  return hipGetLastError();
}

template <bool IsBf16>
hipError_t dispatch(const FwdArgs& a, int64_t r0, hipStream_t s) {
  if (a.d == 128) return launch<IsBf16, 128>(a, r0, s);
  return a.d == 96 ? launch<IsBf16, 96>(a, r0, s) : launch<IsBf16, 64>(a, r0, s);
}

}  // namespace

hipError_t launch_fwd_tail_bf16(const FwdArgs& a, int64_t r0, hipStream_t s) { return dispatch<true>(a, r0, s); }
hipError_t launch_fwd_tail_f16(const FwdArgs& a, int64_t r0, hipStream_t s) { return dispatch<false>(a, r0, s); }

}  // namespace fa
