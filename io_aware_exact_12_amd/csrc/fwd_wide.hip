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
// CU: one wave per SIMD, up to 512 registers a wave.  With no second wave on
// the SIMD, the wave overlaps its own MFMAs and softmax work: key blocks of 32
// rows stream through a 4-stage LDS ring (K and V tiles of 16 KB each, in the
// permuted, swizzled format of the streamed-tile helpers), and block u runs
//   [its row maximum and reference check]  while PV(u-1) drains,
//   [S(u+1) = K Q^T, 16 MFMAs] with the exp2, packing and row sums of P(u)
//                                 placed between them,
//   [O^T += V^T P^T of block u, 16 MFMAs].
// A block's probabilities are taken against the current reference maximum
// without first computing the block's own maximum; only when a lane's partial
// row sum exceeds kSumCap (so some probability may) is the reference raised
// to the running maximum, the 128 accumulators rescaled and the block's
// probabilities formed again.  The result does not depend on the reference,
// which cancels between numerator and denominator.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

#include "fa_internal.hpp"
#include "mfma_common.hpp"
#include "tile_common.hpp"

namespace fa {
namespace {

using namespace mfma;
using namespace tiles;

constexpr float kLn2 = 0.6931471805599453f;
// Cap on a lane's partial row sum of a block (16 probabilities): 2^15 for
// fp16 (its P operand reaches 65504), 2^24 for bf16 (fp32 exponent range;
// bounds |V| by about 2^104 / N so that the fp32 numerator sum stays finite)
template <bool IsBf16> constexpr float kSumCap = IsBf16 ? 16777216.0f : 32768.0f;
// Exponent offset of a row with no reference yet (every key seen so far
// hidden): a visible score then gives probability +inf, so the partial sum
// passes the cap and the block sets the reference; a hidden one gives 0.
constexpr float kNoRef = 1e30f;
constexpr int kB = 32;       // keys per block (one streamed tile)
constexpr int kStages = 4;
constexpr int kAhead = 2;    // LDS operand reads issued this many MFMAs before their use

// A 32-row streamed tile: the first half of STile<D>'s format.
template <int D> struct BlockTile {
  using T = STile<D>;
  static constexpr int kBytes = kB * T::kRowBytes;
  static constexpr int kPerWave = kBytes / 1024 / kW;  // wave-wide 1 KB copies per wave
  static_assert(kPerWave * kW * 1024 == kBytes, "tile copies split evenly over the waves");
  static __device__ __forceinline__ void sources(int wave, int lane, uint32_t row_bytes,
                                                 uint32_t (&src)[kPerWave]) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int byte = (wave + kW * i) * 1024 + 16 * lane;
      const int r = byte / T::kRowBytes, phys = (byte % T::kRowBytes) / 16;
      src[i] = (uint32_t)tile_row(r) * row_bytes + (uint32_t)(16 * (phys ^ T::swz(r)));
    }
  }
};

// MFMA slot of step st (0 scale, 1 exp2, 2 pack and partial sum) of score
// pair e among the kKs score MFMAs of a block (16 at d = 256; 8, 6 or 4 when
// only the values are 256 wide).  Each step lands a few slots after the one
// it depends on.
template <int kKs>
constexpr int slot_of(int e, int st) {
  return kKs == 16 ? e + (st == 0 ? 0 : st == 1 ? 2 : 5)
       : (kKs == 8 || kKs == 6) ? e / 2 + st
                                : (e / 4 + st < 3 ? e / 4 + st : 3);
}

// kWin (causal only): a sliding window of `win` keys, key j visible to query
// i iff i - win < j <= i.  Blocks left of every query's window are skipped
// (the workgroup starts at the first block any of its queries sees, a wave at
// the first its own queries see), and the left-edge mask is applied in the
// blocks that cross a window's start.
// kSparse: a block mask of 64 x 64 blocks (and-ed with causal when that is
// on).  The workgroup lists the 64-key tiles that one of its two 64-row query
// blocks sees and walks their 32-key halves as its blocks; a wave masks the
// blocks of tiles its own query block does not see, and a row that sees no
// key stores O = 0 and LSE = -inf.
// DV is the width of the V and O rows: D = DV = 256, or one of them 256 and
// the other 64, 96 or 128 (plain masks only).
template <bool IsBf16, int D, bool Causal, bool kWin, bool kSparse, int DV = D>
__global__ __launch_bounds__(kThr, 1) void fwd_wide_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int win, int H, int BH, int n_qblocks,
    float c, uint32_t q_sign, Layout lq, Layout in, Layout lv, Layout out,
    const uint8_t* __restrict__ bmask, int64_t m_sb, int64_t m_sh) {
  static_assert(!kWin || Causal, "the sliding window is causal");
  static_assert(!(kWin && kSparse), "one of the two masks");
  static_assert(2 * kB == kSparseBlock && kRes % kSparseBlock == 0, "mask tiles are two blocks");
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using T = STile<D>;
  using BT = BlockTile<D>;
  using BTV = BlockTile<DV>;
  constexpr int kKs = D / 16, kDB = DV / 32;
  constexpr int kStage = BT::kBytes + BTV::kBytes;  // K tile, then V tile
  constexpr int kCopies = BT::kPerWave + BTV::kPerWave;
  static_assert(kCopies <= 15, "the vmcnt wait holds the copies of one block");
  static_assert(kStages * kStage + kSparseBytes <= 160 * 1024, "the ring and the tile list fit the LDS");
  static_assert(DV == D || !(kWin || kSparse), "d_v != d with plain masks only");
  static_assert(kKs == 16 || kKs == 8 || kKs == 6 || kKs == 4, "slot maps exist for 4, 6, 8 and 16 MFMAs");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStage + (kSparse ? kSparseBytes : 0)];

  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (Causal) qb = n_qblocks - 1 - qb;  // heaviest first
  const int b = bh / H, h = bh - b * H;
  const int q0 = qb * kRes, qw0 = q0 + 32 * wave, my_q = qw0 + l32;

  vec8 qf[kKs];
  load_resident<IsBf16, D>(qf, Q + (b * lq.sb + h * lq.sh), N, my_q, lq.sn, g, q_sign);

  // blocks of the workgroup, and the last one this wave computes
  const int last_row = min(N, q0 + kRes) - 1;
  int n_blk = Causal ? last_row / kB + 1 : (N + kB - 1) / kB;
  const bool wave_live = qw0 < N;
  // block-sparse: the listed tiles (index | query-block bits << 16) in LDS
  uint32_t* const list = reinterpret_cast<uint32_t*>(smem + kStages * kStage);
  const int n_tiles_all = (N + kSparseBlock - 1) / kSparseBlock;
  int n_pos = 0;
  if constexpr (kSparse) {
    const int qb0 = q0 / kSparseBlock;
    const int n_tiles = Causal ? last_row / kSparseBlock + 1 : n_tiles_all;
    const uint8_t* mk = bmask + (bh / H) * m_sb + (bh % H) * m_sh;
    n_pos = compact_tiles<kW>(list, n_tiles, [&](int jt) {
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < kRes / kSparseBlock; ++i) {
        const int qbk = qb0 + i;
        if (qbk < n_tiles_all && (!Causal || jt <= qbk) && mk[(int64_t)qbk * n_tiles_all + jt] != 0)
          bits |= 1u << i;
      }
      return bits;
    });
    n_blk = 2 * n_pos;
  }
  // first key of block u (block-sparse: half u & 1 of the tile at list
  // position u / 2; past the list, a tile past the end, which reads as zeros)
  auto ks_of = [&](int u) {
    if constexpr (kSparse) {
      const int p = u >> 1;
      const int t = p < n_pos ? __builtin_amdgcn_readfirstlane((int)(list[p] & 0xFFFFu)) : n_tiles_all;
      return kSparseBlock * t + kB * (u & 1);
    } else {
      return u * kB;
    }
  };
  const int u_last = (Causal && !kSparse) ? min(qw0 + 31, N - 1) / kB : n_blk - 1;
  // first block of the workgroup and of this wave (sliding window; 0 without)
  const int u_first = kWin ? max(0, q0 - win + 1) / kB : 0;
  const int u_lo = kWin ? max(0, qw0 - win + 1) / kB : 0;
  if constexpr (DV == D) lv = in;  // one layout: the d_v addressing folds away
  const uint16_t* k_h = K + (b * in.sb + h * in.sh);
  const uint16_t* v_h = V + (b * lv.sb + h * lv.sh);
  uint32_t src[BT::kPerWave], src_v[BTV::kPerWave];
  BT::sources(wave, lane, (uint32_t)(2 * in.sn), src);
  BTV::sources(wave, lane, (uint32_t)(2 * lv.sn), src_v);
  const uint32_t lds0 = lds_u32(smem);
  // copies of block u's K and V rows into its stage: kCopies per wave, K's
  // first.  A block past the last one gets empty buffer ranges: its copies
  // read nothing and land in the stage that no wave reads any more.
  struct Copies {
    i32x4 rk, rv;
    uint32_t base;
  };
  auto prepare = [&](int u, bool real) {
    const int row0 = ks_of(u), left = real ? N - row0 : 0;
    const uint32_t kbytes =
        left > 0 ? (uint32_t)(left - 1) * (uint32_t)(2 * in.sn) + (uint32_t)T::kDataBytes : 0u;
    const uint32_t vbytes =
        left > 0 ? (uint32_t)(left - 1) * (uint32_t)(2 * lv.sn) + (uint32_t)STile<DV>::kDataBytes : 0u;
    Copies cp;
    cp.rk = make_rsrc(k_h + (int64_t)row0 * in.sn, kbytes);
    cp.rv = make_rsrc(v_h + (int64_t)row0 * lv.sn, vbytes);
    cp.base = lds0 + (uint32_t)((u & (kStages - 1)) * kStage);
    return cp;
  };
  auto copy = [&](const Copies& cp, int i) {
    if (i < BT::kPerWave)
      dma16(cp.rk, cp.base + (uint32_t)((wave + kW * i) * 1024), src[i]);
    else
      dma16(cp.rv, cp.base + (uint32_t)(BT::kBytes + (wave + kW * (i - BT::kPerWave)) * 1024),
            src_v[i - BT::kPerWave]);
  };
  auto issue = [&](int u) {
    const Copies cp = prepare(u, true);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy(cp, i);
  };
  auto k_tile = [&](int u) { return smem + (u & (kStages - 1)) * kStage; };
  auto v_tile = [&](int u) { return smem + (u & (kStages - 1)) * kStage + BT::kBytes; };

  f32x16 acc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) acc[i] = f32x16{};
  float m = -INFINITY;  // reference: raw (sign-adjusted) score of this lane's query
  float neg_mc = kNoRef;  // -m * c, or kNoRef while m = -inf
  float l = 0.f;        // this lane half's share of the row sum, relative to m
  f32x16 s_cur = f32x16{}, s_next = f32x16{};

  for (int u = u_first; u < u_first + kStages - 1 && u < n_blk; ++u) issue(u);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  // scores of the first block of every wave that starts in the workgroup's
  // first block (all of them without a window); K tile u_first is resident
  auto first_scores = [&](int u) {
    const uint8_t* kt = k_tile(u);
    f32x16 st = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk) st = E::mfma(row_frag<IsBf16, D>(kt, l32, g, kk), qf[kk], st);
    return st;
  };
  if (wave_live && u_lo == u_first) s_cur = first_scores(u_first);

  for (int u = u_first; u < n_blk; ++u) {
    // block u+3 goes into the stage block u-1 left.  A wave that computes
    // block u spreads its copies over the score MFMAs, so that the texture
    // unit moves them while the matrix cores work; the others issue them at
    // once.
    const Copies cp = prepare(u + kStages - 1, u + kStages - 1 < n_blk);
    const bool busy = wave_live && u >= u_lo && u <= u_last;
    if (!busy) {
#pragma unroll
      for (int i = 0; i < kCopies; ++i) copy(cp, i);
    }
    // a wave whose window starts after the workgroup's first block forms the
    // scores of its first block from the resident tile
    if (kWin && wave_live && u == u_lo && u_lo > u_first) s_cur = first_scores(u);
    if (busy) {
      const int ks0 = ks_of(u);
      // register rr of lane half g holds key ks0 + 16 (rr >> 3) + 8 g + (rr & 7)
      if (kSparse && ((list[u >> 1] >> (16 + wave / 2)) & 1u) == 0) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) s_cur[rr] = -INFINITY;  // tile hidden from this query block
      } else if ((Causal && ks0 + kB - 1 > qw0) || ks0 + kB > N || (kWin && ks0 <= qw0 + 31 - win)) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int kj = ks0 + 16 * (rr >> 3) + 8 * g + (rr & 7);
          if (kj >= N || (Causal && kj > my_q) || (kWin && kj <= my_q - win)) s_cur[rr] = -INFINITY;
        }
      }

      // S(u+1) with P(u) between its MFMAs; a wave's last block forms no S
      // (two copies of the loop, so that no branch sits between the MFMAs)
      u32x4 pw[2];
      float sum[2] = {0.f, 0.f};
      // the first V^T operands of the PV MFMAs below are read two score MFMAs
      // before the score phase ends (block u's V tile is resident), so the
      // PV phase does not start on an LDS wait
      const uint8_t* vt = v_tile(u);
      vec8 va[kAhead];
      auto phase_a = [&](auto next) {
        constexpr bool kNext = decltype(next)::value;
        const uint8_t* kt = k_tile(u + 1);
        float pr[16];
        vec8 ka[kAhead];
        if constexpr (kNext) {
#pragma unroll
          for (int r = 0; r < kAhead && r < kKs; ++r) ka[r] = row_frag<IsBf16, D>(kt, l32, g, r);
        }
#pragma unroll
        for (int t = 0; t < kKs; ++t) {
#pragma unroll
          for (int i = 0; i < kCopies; ++i)
            if (t == i * kKs / kCopies) copy(cp, i);
          if constexpr (kNext) {
            s_next = E::mfma(ka[t % kAhead], qf[t], t == 0 ? f32x16{} : s_next);
            if (t + kAhead < kKs) ka[t % kAhead] = row_frag<IsBf16, D>(kt, l32, g, t + kAhead);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (t == slot_of<kKs>(e, 0)) {
              pr[2 * e] = __builtin_fmaf(s_cur[2 * e], c, neg_mc);
              pr[2 * e + 1] = __builtin_fmaf(s_cur[2 * e + 1], c, neg_mc);
            }
            if (t == slot_of<kKs>(e, 1)) {
              pr[2 * e] = __builtin_amdgcn_exp2f(pr[2 * e]);
              pr[2 * e + 1] = __builtin_amdgcn_exp2f(pr[2 * e + 1]);
            }
            if (t == slot_of<kKs>(e, 2)) {
              pw[e >> 2][e & 3] = E::pack2(pr[2 * e], pr[2 * e + 1]);
              sum[e & 1] += pr[2 * e] + pr[2 * e + 1];
            }
          }
          if (t == (kKs >= 2 ? kKs - 2 : 0)) {
#pragma unroll
            for (int r = 0; r < kAhead && r < 2 * kDB; ++r) va[r] = tr_frag<IsBf16, DV>(vt, lane, r / kDB, r % kDB);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (u + 1 <= u_last)
        phase_a(std::true_type{});
      else
        phase_a(std::false_type{});
      // Keep the packing inside the MFMA stream (the rare path below
      // overwrites pw; without this use the compiler sinks the conversions
      // past its branch).
      asm volatile("" ::"v"(pw[0]), "v"(pw[1]));
      if (__builtin_amdgcn_ballot_w64(sum[0] + sum[1] > kSumCap<IsBf16>) != 0) {
        // rare: raise the reference to the running maximum over both lane
        // halves, rescale l and a, and take this block's probabilities again.
        // A row whose block shows no key keeps m = -inf and kNoRef.
        float mx = s_cur[0];
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, s_cur[rr]);
        const float m_new = fmaxf(m, xhalf_max(mx));
        const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db) acc[db] *= alpha;
        m = m_new;
        neg_mc = m_new == -INFINITY ? kNoRef : -m_new * c;
        sum[0] = sum[1] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[2 * e], c, neg_mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[2 * e + 1], c, neg_mc));
          pw[e >> 2][e & 3] = E::pack2(p0, p1);
          sum[e & 1] += p0 + p1;
        }
      }
      l += sum[0] + sum[1];

      // O^T += V^T P^T of block u; operand reads two MFMAs ahead
#pragma unroll
      for (int i = 0; i < 2 * kDB; ++i) {
        const int tt = i / kDB, db = i % kDB;
        acc[db] = E::mfma(va[i % kAhead], __builtin_bit_cast(vec8, pw[tt]), acc[db]);
        if (i + kAhead < 2 * kDB)
          va[i % kAhead] = tr_frag<IsBf16, DV>(vt, lane, (i + kAhead) / kDB, (i + kAhead) % kDB);
        __builtin_amdgcn_sched_barrier(0);
      }
      s_cur = s_next;
    }
    // block u+2's tiles must be in LDS for S(u+2) in the next block; the
    // copies just issued (block u+3) may stay in flight until then, and all
    // are done before the last barrier
    if (u + 1 < n_blk)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kCopies);  // the latest block's copies
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if (!wave_live) return;
  const float l_tot = xhalf_sum(l);
  if (my_q >= N) return;
  const float inv = (!kSparse || l_tot > 0.f) ? 1.0f / l_tot : 0.f;  // a row with no key: O = 0
  store_row<IsBf16, DV>(O + (b * out.sb + h * out.sh), my_q, out.sn, g, acc, inv);
  if (LSE != nullptr && g == 0)
    LSE[(int64_t)bh * N + my_q] = ((m == -INFINITY ? 0.f : m * c) + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <bool IsBf16, int D, bool Causal, bool kWin = false, bool kSparse = false, int DV = D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int N = (int)a.N;
  const int BH = (int)(a.B * a.H);
  const int n_qblocks = (N + kRes - 1) / kRes;
  // c = |scale| * log2(e); a zero scale is run as the limit scale -> 0+ (every
  // exp2 argument rounds to 0, so visible keys weigh exactly 1)
  const float c = a.scale != 0.f ? __builtin_fabsf(a.scale) * 1.4426950408889634f : 1e-30f;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const int win = (int)(a.window < a.N ? a.window : a.N);
  hipLaunchKernelGGL((fwd_wide_kernel<IsBf16, D, Causal, kWin, kSparse, DV>), dim3((unsigned)(n_qblocks * BH)),
                     dim3(kThr), 0, stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<uint16_t*>(a.o), a.lse, N, win, (int)a.H, BH, n_qblocks, c, q_sign, a.lq,
                     a.in, a.lv, a.out, a.block_mask, a.mask_sb, a.mask_sh);
  return hipGetLastError();
}

template <bool IsBf16, int D, int DV>
hipError_t launch_dv(const FwdArgs& a, hipStream_t s) {
  return a.causal ? launch<IsBf16, D, true, false, false, DV>(a, s) : launch<IsBf16, D, false, false, false, DV>(a, s);
}

template <bool IsBf16>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
  // d_v != d with one of them 256 (plain masks only)
  if (a.dv != a.d) {
    if (a.d == 256)
      return a.dv == 64 ? launch_dv<IsBf16, 256, 64>(a, s)
           : a.dv == 96 ? launch_dv<IsBf16, 256, 96>(a, s) : launch_dv<IsBf16, 256, 128>(a, s);
    return a.d == 64 ? launch_dv<IsBf16, 64, 256>(a, s)
         : a.d == 96 ? launch_dv<IsBf16, 96, 256>(a, s) : launch_dv<IsBf16, 128, 256>(a, s);
  }
  if (a.block_mask != nullptr)
    return a.causal ? launch<IsBf16, 256, true, false, true>(a, s) : launch<IsBf16, 256, false, false, true>(a, s);
  if (!a.causal) return launch<IsBf16, 256, false>(a, s);
  if (a.window < a.N) return launch<IsBf16, 256, true, true>(a, s);
  return launch<IsBf16, 256, true>(a, s);
}

}  // namespace

hipError_t launch_fwd_wide_bf16(const FwdArgs& a, hipStream_t s) { return dispatch<true>(a, s); }
hipError_t launch_fwd_wide_f16(const FwdArgs& a, hipStream_t s) { return dispatch<false>(a, s); }

}  // namespace fa
