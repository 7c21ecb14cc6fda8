// Exact attention forward for fp32 inputs on gfx950.
//
// The fp32 path is held to a 1e-5 absolute error, also for sharp softmax rows
// where a score of magnitude ~30 rounded to fp32 would already move exp() by
// ~2e-6 relative.  So the scores, the running maximum, the exponentials and
// the denominator are carried in fp64 (products of fp32 inputs are exact in
// fp64), while the d-wide numerator is accumulated in fp32 from the same
// fp32-rounded probabilities and rescale factors that enter the denominator,
// so that their ratio does not drift.  Same schedule as the MFMA path -- query
// rows resident, key/value tiles streamed through LDS, a running
// (max, denominator, unnormalised numerator) per row rescaled by
// alpha = exp(m_old - m_new) ("Flash Attention: IO-Aware Exact Attention",
// section "Online softmax makes tiling exact") -- with one query row per lane
// and scalar arithmetic.  It is the small-size, high-precision path, not a
// throughput path.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (one row per lane of each wave)
constexpr int kKeys = 16;   // keys per LDS tile
constexpr int kSplit = 4;   // waves per workgroup; wave w takes key tiles w, w + kSplit, ..
// Below this many 64-row workgroups (one per CU of MI355X) the launch runs the
// row-per-wave kernel instead.
constexpr int64_t kRowKernelBelow = 256;

// The rows' key range is split over kSplit waves, each with its own LDS tiles
// and its own running (max, denominator, numerator) state; the states are
// merged at the end with the same alpha rescaling, in wave order, so the
// result is deterministic.
template <int D, int DV, bool Causal>
__global__ __launch_bounds__(kRows * kSplit) void fwd_f32_kernel(const float* __restrict__ Q,
                                                                 const float* __restrict__ K,
                                                                 const float* __restrict__ V,
                                                                 float* __restrict__ O,
                                                                 float* __restrict__ LSE, int N,
                                                                 int win, int H, int n_qblocks, float scale,
                                                                 Layout lq, Layout in, Layout lv, Layout out,
                                                                 const uint8_t* __restrict__ bmask,
                                                                 int64_t m_sb, int64_t m_sh) {
  constexpr int kQStride = D + 1;  // odd stride: lanes reading their own row hit distinct banks
  constexpr int kAStride = DV + 1;
  static_assert(kRows * kAStride <= kSplit * kKeys * (D + DV), "the merge buffer fits in the tiles");
  __shared__ float qs[kRows * kQStride];
  __shared__ __attribute__((aligned(16))) float tiles[kSplit * kKeys * (D + DV)];
  __shared__ double part_m[kSplit][kRows], part_l[kSplit][kRows];

  const int lane = threadIdx.x & (kRows - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kRows);
  float* ks = tiles + wave * kKeys * (D + DV);
  float* vs = ks + kKeys * D;
  const int bh = blockIdx.x / n_qblocks;
  const int q0 = (blockIdx.x % n_qblocks) * kRows;
  const int b = bh / H, h = bh - b * H;
  const int64_t head_off = b * in.sb + h * in.sh;
  const int64_t sn = in.sn;
  const float* Qh = Q + (b * lq.sb + h * lq.sh);
  const float* Kh = K + head_off;
  const float* Vh = V + (b * lv.sb + h * lv.sh);

  for (int idx = threadIdx.x; idx < kRows * D; idx += kRows * kSplit) {
    const int r = idx / D, col = idx % D;
    qs[r * kQStride + col] = (q0 + r < N) ? Qh[(int64_t)(q0 + r) * lq.sn + col] : 0.f;
  }
  __syncthreads();

  const int my_q = q0 + lane;
  // block-sparse mask row of this query (64 x 64 blocks), if any
  const int n_kb = (N + 63) / 64;
  const uint8_t* mrow = (bmask != nullptr && my_q < N)
                            ? bmask + b * m_sb + h * m_sh + (int64_t)(my_q / 64) * n_kb
                            : nullptr;
  const int last_row = min(N, q0 + kRows) - 1;
  const int n_keys = Causal ? last_row + 1 : N;
  // first key any row of the block can see (sliding window; 0 without one)
  const int key_lo = Causal ? max(0, q0 - win + 1) / kKeys * kKeys : 0;

  float acc[DV];
#pragma unroll
  for (int i = 0; i < DV; ++i) acc[i] = 0.f;
  double m_run = -INFINITY, l_run = 0.0;
  const double dscale = (double)scale;

  // Each wave reads only the tiles it wrote itself, and a wave's LDS accesses
  // complete in order, so the waves need no barrier inside the loop.
  for (int key0 = key_lo + wave * kKeys; key0 < n_keys; key0 += kSplit * kKeys) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int idx = lane; idx < kKeys * D / 4; idx += kRows) {
      const int r = (idx * 4) / D, col = (idx * 4) % D;
      const bool ok = key0 + r < N;
      const float4 kv = ok ? *reinterpret_cast<const float4*>(Kh + (int64_t)(key0 + r) * sn + col)
                           : float4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<float4*>(ks + r * D + col) = kv;
    }
    for (int idx = lane; idx < kKeys * DV / 4; idx += kRows) {
      const int r = (idx * 4) / DV, col = (idx * 4) % DV;
      const bool ok = key0 + r < N;
      const float4 vv = ok ? *reinterpret_cast<const float4*>(Vh + (int64_t)(key0 + r) * lv.sn + col)
                           : float4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<float4*>(vs + r * DV + col) = vv;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();

    double t[kKeys];
#pragma unroll
    for (int j = 0; j < kKeys; ++j) t[j] = 0.0;
    for (int col = 0; col < D; ++col) {
      const double qv = (double)qs[lane * kQStride + col];
#pragma unroll
      for (int j = 0; j < kKeys; ++j) t[j] = __builtin_fma(qv, (double)ks[j * D + col], t[j]);
    }
    double tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const int key = key0 + j;
      const bool hide = key >= N || (Causal && (key > my_q || key <= my_q - win)) ||
                        (bmask != nullptr && (mrow == nullptr || mrow[key / 64] == 0));
      t[j] = hide ? -INFINITY : t[j] * dscale;
      tmax = fmax(tmax, t[j]);
    }
    const double m_new = fmax(m_run, tmax);
    if (m_new == -INFINITY) continue;  // no visible key yet: state unchanged
    const float alpha = (m_run == -INFINITY) ? 0.f : (float)exp(m_run - m_new);
    float p[kKeys];
    double psum = 0.0;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      p[j] = (t[j] == -INFINITY) ? 0.f : (float)exp(t[j] - m_new);
      psum += (double)p[j];
    }
    l_run = (double)alpha * l_run + psum;
    m_run = m_new;
#pragma unroll
    for (int col = 0; col < DV; ++col) {
      float a = alpha * acc[col];
#pragma unroll
      for (int j = 0; j < kKeys; ++j) a = __builtin_fmaf(p[j], vs[j * DV + col], a);
      acc[col] = a;
    }
  }

  // Merge: m = max over the waves, alpha_w = exp(m_w - m) rounded to fp32 and
  // used for both the denominator and the numerator; the numerators are
  // added into LDS in wave order.
  part_m[wave][lane] = m_run;
  part_l[wave][lane] = l_run;
  __syncthreads();
  double m_all = -INFINITY;
#pragma unroll
  for (int w = 0; w < kSplit; ++w) m_all = fmax(m_all, part_m[w][lane]);
  double l_all = 0.0;
  float alpha_me = 0.f;
#pragma unroll
  for (int w = 0; w < kSplit; ++w) {
    const double mw = part_m[w][lane];
    const float aw = (mw == -INFINITY) ? 0.f : (float)exp(mw - m_all);
    l_all += (double)aw * part_l[w][lane];
    if (w == wave) alpha_me = aw;
  }
  float* sum = tiles;  // [kRows][kAStride]; every wave is past its last tile read
  for (int w = 0; w < kSplit; ++w) {
    if (w == wave) {
#pragma unroll
      for (int col = 0; col < DV; ++col) {
        const float mine = alpha_me * acc[col];
        sum[lane * kAStride + col] = w == 0 ? mine : sum[lane * kAStride + col] + mine;
      }
    }
    __syncthreads();
  }
  if (wave != 0 || my_q >= N) return;
  float* orow = O + (b * out.sb + h * out.sh) + (int64_t)my_q * out.sn;
  // a row that saw no key (block-sparse) stores O = 0 and LSE = -inf
#pragma unroll
  for (int col = 0; col < DV; ++col)
    orow[col] = l_all > 0.0 ? (float)((double)sum[lane * kAStride + col] / l_all) : 0.f;
  if (LSE != nullptr) LSE[(int64_t)bh * N + my_q] = (float)(m_all + log(l_all));
}

// Launches too small to fill the GPU with 64-row workgroups (fewer than 256
// of them): one workgroup per query row instead, whose four waves take the
// row's 64-key blocks in turn (wave w: blocks w, w + 4, ..), so that even a
// single 256-row head spreads over every CU.  Per block a wave forms the
// scores with one key per lane (fp64 dot products of the fp32 inputs, as
// above), takes the block maximum and the sum of the fp32-rounded
// probabilities with XOR butterflies (every lane ends with the same bits), and
// accumulates the numerator with one output column per lane, in key order,
// from the probabilities it left in LDS.  The four running states merge at the
// end as in the kernel above: alpha_w = exp(m_w - m) rounded to fp32 for both
// the denominator and the numerator, added in wave order.
constexpr int kRowWaves = 4;

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int D, int DV, bool Causal>
__global__ __launch_bounds__(64 * kRowWaves) void fwd_f32_row_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int win, int H, float scale, Layout lq,
    Layout in, Layout lv, Layout out, const uint8_t* __restrict__ bmask, int64_t m_sb, int64_t m_sh) {
  constexpr int kCols = (DV + 63) / 64;  // numerator columns per lane
  __shared__ float pbuf[kRowWaves][64];
  __shared__ float part_acc[kRowWaves][DV];
  __shared__ double part_m[kRowWaves], part_l[kRowWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = (int)(blockIdx.x / (unsigned)N), i = (int)(blockIdx.x % (unsigned)N);
  const int b = bh / H, h = bh - b * H;
  const float* qrow = Q + (b * lq.sb + h * lq.sh) + (int64_t)i * lq.sn;
  const float* Kh = K + (b * in.sb + h * in.sh);
  const float* Vh = V + (b * lv.sb + h * lv.sh);
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = qrow[d];
  // visible keys lo .. hi - 1 (causal, sliding window), in blocks of 64
  const int lo = Causal ? max(0, i - win + 1) : 0;
  const int hi = Causal ? i + 1 : N;
  const int n_kb = (N + 63) / 64;
  const uint8_t* mrow = bmask != nullptr ? bmask + b * m_sb + h * m_sh + (int64_t)(i / 64) * n_kb : nullptr;
  const double dscale = (double)scale;
  double m_run = -INFINITY, l_run = 0.0;
  float acc[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) acc[c] = 0.f;

  for (int kb = (lo & ~63) + 64 * wave; kb < hi; kb += 64 * kRowWaves) {
    if (mrow != nullptr && mrow[kb / 64] == 0) continue;  // a hidden 64 x 64 block
    const int j = kb + lane;
    const bool vis = j >= lo && j < hi;
    double s = 0.0;
    if (vis) {
      const float* kr = Kh + (int64_t)j * in.sn;
#pragma unroll
      for (int d = 0; d < D; ++d) s = __builtin_fma((double)q[d], (double)kr[d], s);
    }
    const double t = vis ? s * dscale : -INFINITY;
    const double m_new = fmax(m_run, wave_max(t));
    if (m_new == -INFINITY) continue;  // no visible key yet: state unchanged
    const float alpha = (m_run == -INFINITY) ? 0.f : (float)exp(m_run - m_new);
    const float p = vis ? (float)exp(t - m_new) : 0.f;
    l_run = (double)alpha * l_run + wave_sum((double)p);
    m_run = m_new;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    pbuf[wave][lane] = p;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int nk = min(64, hi - kb);  // keys of the block that exist and may be visible
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      const int col = lane + 64 * c;
      if (col < DV) {
        float a = alpha * acc[c];
        const float* vcol = Vh + col;
        // eight value loads in flight at a time; rows past the block's last
        // existing key read that key's row and are not added
#pragma unroll
        for (int j0 = 0; j0 < 64; j0 += 8) {
          float vv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) vv[u] = vcol[(int64_t)(kb + min(j0 + u, nk - 1)) * lv.sn];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (j0 + u < nk) a = __builtin_fmaf(pbuf[wave][j0 + u], vv[u], a);
        }
        acc[c] = a;
      }
    }
  }
  if (lane == 0) {
    part_m[wave] = m_run;
    part_l[wave] = l_run;
  }
#pragma unroll
  for (int c = 0; c < kCols; ++c)
    if (lane + 64 * c < DV) part_acc[wave][lane + 64 * c] = acc[c];
  __syncthreads();
  if (wave != 0) return;
  double m_all = -INFINITY;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) m_all = fmax(m_all, part_m[w]);
  double l_all = 0.0;
  float aw[kRowWaves];
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    aw[w] = part_m[w] == -INFINITY ? 0.f : (float)exp(part_m[w] - m_all);
    l_all += (double)aw[w] * part_l[w];
  }
  float* orow = O + (b * out.sb + h * out.sh) + (int64_t)i * out.sn;
  // a row that saw no key (block-sparse) stores O = 0 and LSE = -inf
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int col = lane + 64 * c;
    if (col < DV) {
      float sum = aw[0] * part_acc[0][col];
#pragma unroll
      for (int w = 1; w < kRowWaves; ++w) sum += aw[w] * part_acc[w][col];
      orow[col] = l_all > 0.0 ? (float)((double)sum / l_all) : 0.f;
    }
  }
  if (LSE != nullptr && lane == 0) LSE[(int64_t)bh * N + i] = (float)(m_all + log(l_all));
}

template <int D, bool Causal, int DV = D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int N = (int)a.N;
  const int n_qblocks = (N + kRows - 1) / kRows;
  const int64_t BH = a.B * a.H;
  if (n_qblocks * BH < kRowKernelBelow) {
    // one workgroup per query row: fewer than 256 * 64 rows here
    hipLaunchKernelGGL((fwd_f32_row_kernel<D, DV, Causal>), dim3((unsigned)(BH * N)), dim3(64 * kRowWaves), 0,
                       stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, N,
                       (int)(a.window < a.N ? a.window : a.N), (int)a.H, a.scale, a.lq, a.in, a.lv, a.out,
                       a.block_mask, a.mask_sb, a.mask_sh);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(n_qblocks * a.B * a.H));
  hipLaunchKernelGGL((fwd_f32_kernel<D, DV, Causal>), grid, dim3(kRows * kSplit), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, N,
                     (int)(a.window < a.N ? a.window : a.N), (int)a.H, n_qblocks, a.scale, a.lq, a.in, a.lv, a.out,
                     a.block_mask, a.mask_sb, a.mask_sh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  // d_v != d: d, d_v in {64, 96, 128}
  if (a.dv != a.d) {
    if (a.d == 128)
      return a.dv == 64 ? (a.causal ? launch<128, true, 64>(a, s) : launch<128, false, 64>(a, s))
                        : (a.causal ? launch<128, true, 96>(a, s) : launch<128, false, 96>(a, s));
    if (a.d == 96)
      return a.dv == 64 ? (a.causal ? launch<96, true, 64>(a, s) : launch<96, false, 64>(a, s))
                        : (a.causal ? launch<96, true, 128>(a, s) : launch<96, false, 128>(a, s));
    return a.dv == 96 ? (a.causal ? launch<64, true, 96>(a, s) : launch<64, false, 96>(a, s))
                      : (a.causal ? launch<64, true, 128>(a, s) : launch<64, false, 128>(a, s));
  }
  if (a.d == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
  if (a.d == 96) return a.causal ? launch<96, true>(a, s) : launch<96, false>(a, s);
  return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace fa
