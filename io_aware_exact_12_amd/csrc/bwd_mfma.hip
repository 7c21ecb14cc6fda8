// Exact attention backward for bf16 / fp16 on gfx950 (MI355X), using MFMA.
//
// The forward pass keeps only O and the per-row log-sum-exp; the backward pass
// recomputes each tile of scores and probabilities from Q, K and that
// statistic instead of reading a stored N x N matrix ("Flash Attention:
// IO-Aware Exact Attention", section "Storage, arithmetic and IO are separate
// quantities"; Road to Intelligence "FlashAttention", section "The trick that
// makes tiling possible").  With S = scale Q K^T, P = exp(S - LSE) and dO the
// output gradient, the gradient of a row softmax followed by P V is
//
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
//     dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q.
//
// D_i equals sum_j P_ij dP_ij.  Computing it as rowsum(dO * O) from the
// stored low-precision O puts O's rounding (2^-9 relative in bf16) straight
// into dS = P (dP - D), where dP and D nearly cancel on a row's dominant
// keys; so D is formed from the recomputed P and dP in fp32 instead.
//
// Two kernels per call, whose sums run in a fixed order, so the result is deterministic
// (the only atomic is the block-sparse split path's per-key-block counter,
// which picks the workgroup that adds the partial sums, in chunk order):
//   * bwd_dq:     a workgroup keeps 128 query rows resident (Q^T and dO^T in
//                 registers) and streams 64-key tiles of K and V through LDS
//                 twice: pass 1 accumulates D = sum_j P dP and stores it in
//                 the caller's workspace, pass 2 accumulates dQ^T;
//   * bwd_dkdv:   a workgroup keeps 128 keys resident (K^T and V^T as MFMA
//                 operands in registers, dK^T and dV^T accumulated in
//                 registers) and streams 64-query tiles of Q, dO, LSE and D
//                 through LDS.  It runs after bwd_dq on the same stream.
// For d = d_v <= 128 under plain and sliding-window masks, each of the two
// runs as a wave-pair kernel instead (bwd_dq_pair, bwd_dkdv_pair): the two
// waves of a SIMD share 32 resident rows and split each streamed tile's
// products between them, so S is formed once per (query, key) pair in each
// kernel and every tile streams once.  bwd_dq_pair forms dQ in one pass from
// D~ = rowsum(dO * O) and corrects it with the exact D at the end (the
// identity is stated at the kernel).
// All of them use the 32x32x16 MFMA with the resident index in the lane
// column, so per-row (or per-key) scalars stay lane-local.  Tile rows are
// stored in LDS in the permuted order that makes a 32-row block's MFMA output
// hold 8 consecutive rows per lane half, so P and dS are reused as MFMA
// operands straight from registers; the transposed operands (Q^T, dO^T, K^T)
// come from the gfx950 LDS transpose read.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "fa_internal.hpp"
#include "mfma_common.hpp"
#include "tile_common.hpp"

namespace fa {
namespace {

using namespace mfma;
using namespace tiles;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// ---------------------------------------------------------------- dK, dV
// Per wave: 32 resident keys kw0 .. kw0 + 31 (lane column = key).  Query tiles
// of 64 rows (Q, dO, -LSE log2 e, D) stream through two LDS stages; the copies
// of tile it + 1 are issued before tile it is computed.  Two passes over the
// tiles, so that only one set of accumulators is live at a time (the kernel
// then fits two waves per SIMD).  For each 32-query half:
//   pass V:  S = Q K^T, P = exp2(c S - LSE2), dV^T += dO^T P
//   pass K:  S, dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS
// (A = Q / dO rows from LDS or dO^T / Q^T by transpose reads, B = K^T / V^T
// resident or P / dS from registers; query in the register index).  Masks
// (causal diagonal, sequence ends) are applied only in tiles that can need
// them; a half of a masked tile that lies before all of the wave's keys still
// runs and contributes zeros.  A negative scale flips the sign of the resident
// K (exact), so S carries the sign and dK = scale dS^T Q uses Q as stored.
template <int D, int DV = D> struct DkdvLds {
  static constexpr int kQ = 0;
  static constexpr int kDO = STile<D>::kBytes;                     // dO rows of d_v
  static constexpr int kLse = kDO + STile<DV>::kBytes;  // -LSE * log2(e) of the 64 queries
  static constexpr int kD = kLse + 4 * kT;
  static constexpr int kStage = kD + 4 * kT;
  static constexpr int kBytes = 2 * kStage;
};

template <bool IsBf16, int D, bool Causal, int Mode, int DV = D>
struct DkdvBlock {
  static constexpr bool kWin = Causal && Mode == kModeWindow;  // sliding window narrower than N
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using T = STile<D>;    // Q tiles
  using TO = STile<DV>;  // dO tiles (d_v wide)
  using Ld = DkdvLds<D, DV>;
  static constexpr int kKs = D / 16, kDB = D / 32;      // over d: S = Q K^T, dK^T
  static constexpr int kKsO = DV / 16, kDBO = DV / 32;  // over d_v: dP = dO V^T, dV^T
  static constexpr int kDBA = kDB > kDBO ? kDB : kDBO;
  static constexpr int kMin = kKs < kKsO ? kKs : kKsO;
  // Rows of 32 chunks (d = 256): the swizzle (< 16) never moves a chunk
  // between the two 256-byte halves of a row, so the offsets of the second
  // half are those of the first plus 256 and only the first half's are kept.
  static constexpr int kRo = kKs > 8 ? 8 : kKs, kTo = kDB > 4 ? 4 : kDB;

  int lane, g, N, win, my_k;
  float c;
  vec8 kf[kKs], vf[kKsO];
  f32x16 acc[kDBA];       // dV^T in pass V, dK^T in pass K
  int roff[kRo], roffO[kKsO];    // row operand of k step kk: LDS row l32, chunk 2 kk + g
  int toff[2][kTo], toffO[2][kDBO];  // transpose reads (elements 0..3 / 4..7) of d block db

  __device__ __forceinline__ void init(int lane_, int N_, int win_, int kw0, float c_) {
    lane = lane_;
    N = N_;
    win = win_;
    c = c_;
    g = lane >> 5;
    my_k = kw0 + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < kRo; ++kk) roff[kk] = T::at(lane & 31, 2 * kk + g);
    if constexpr (DV != D) {
#pragma unroll
      for (int kk = 0; kk < kKsO; ++kk) roffO[kk] = TO::at(lane & 31, 2 * kk + g);
    }
    const int grp = lane >> 4, s16 = lane & 15;
    const int r0 = 4 * g + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < kTo; ++db) {
      const int col = 2 * (16 * (grp & 1) + 4 * (s16 & 3)) + 64 * db;  // byte column
      toff[0][db] = T::at(r0, col >> 4) + (col & 15);
      toff[1][db] = T::at(r0 + 8, col >> 4) + (col & 15);
    }
    if constexpr (DV != D) {
#pragma unroll
      for (int db = 0; db < kDBO; ++db) {
        const int col = 2 * (16 * (grp & 1) + 4 * (s16 & 3)) + 64 * db;
        toffO[0][db] = TO::at(r0, col >> 4) + (col & 15);
        toffO[1][db] = TO::at(r0 + 8, col >> 4) + (col & 15);
      }
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kDBA; ++i) acc[i] = f32x16{};
  }

  // Logical tile rows 16 t + 32 h keep their swizzle, so a half and a k step
  // only add whole-row offsets to the per-lane offsets above.
  __device__ __forceinline__ vec8 row_op(const uint8_t* tile, int h, int kk) const {
    return *reinterpret_cast<const vec8*>(tile + roff[kk % kRo] + 256 * (kk / kRo) + 32 * h * T::kRowBytes);
  }
  __device__ __forceinline__ vec8 tr_op(const uint8_t* tile, int h, int t, int db) const {
    const uint8_t* p = tile + (32 * h + 16 * t) * T::kRowBytes + 256 * (db / kTo);
    const auto lo = E::read_tr((const lds_void*)(p + toff[0][db % kTo]));
    const auto hi = E::read_tr((const lds_void*)(p + toff[1][db % kTo]));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // the same two reads on a dO tile (d_v wide)
  __device__ __forceinline__ vec8 row_opO(const uint8_t* tile, int h, int kk) const {
    if constexpr (DV == D) return row_op(tile, h, kk);
    return *reinterpret_cast<const vec8*>(tile + roffO[kk] + 32 * h * TO::kRowBytes);
  }
  __device__ __forceinline__ vec8 tr_opO(const uint8_t* tile, int h, int t, int db) const {
    if constexpr (DV == D) return tr_op(tile, h, t, db);
    const uint8_t* p = tile + (32 * h + 16 * t) * TO::kRowBytes;
    const auto lo = E::read_tr((const lds_void*)(p + toffO[0][db]));
    const auto hi = E::read_tr((const lds_void*)(p + toffO[1][db]));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // MFMA i of the S / dP chains: while both remain they alternate (S even, dP
  // odd); the longer chain then finishes alone
  static constexpr bool is_dp(int i) { return i < 2 * kMin ? (i & 1) != 0 : kKsO > kKs; }
  static constexpr int kstep(int i) { return i < 2 * kMin ? i >> 1 : kMin + (i - 2 * kMin); }
  // per-query floats of registers r, r+1 (consecutive queries) of half h
  __device__ __forceinline__ f32x2 pair_vals(const uint8_t* sb, int off, int h, int r) const {
    return *reinterpret_cast<const f32x2*>(reinterpret_cast<const float*>(sb + off) + 32 * h + 8 * g +
                                           16 * (r >> 3) + (r & 7));
  }

  // Probabilities of the 16 registers of a half whose first query is qs0,
  // from nl = -LSE2 of each register's query; with `masked` (wave-uniform:
  // the tile touches the diagonal, a window edge or a sequence end) those of
  // hidden (key, query) pairs are 0.  One code path serves both cases, so the
  // tile loop holds a single copy of the half and no register copies at a join.
  __device__ __forceinline__ void probs(const f32x16& s, const uint8_t* sb, int h, int qs0, bool masked,
                                        float (&p)[16]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x2 nl = pair_vals(sb, Ld::kLse, h, 2 * e);
      p[2 * e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e], c, nl[0]));
      p[2 * e + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * e + 1], c, nl[1]));
    }
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qs0 + 16 * (r >> 3) + 8 * g + (r & 7);
        if ((Causal && my_k > qi) || (kWin && qi >= my_k + win) || qi >= N || my_k >= N) p[r] = 0.f;
      }
    }
  }

  __device__ __forceinline__ void half_v(const uint8_t* sb, int h, int qs0, bool masked) {
    const uint8_t* q = sb + Ld::kQ;
    const uint8_t* o = sb + Ld::kDO;
    // operand reads run two MFMAs ahead; the fences stop the compiler from
    // hoisting all of them (and holding them in registers)
    f32x16 s = f32x16{};
    vec8 a[2] = {row_op(q, h, 0), row_op(q, h, 1)};
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk) {
      s = E::mfma(a[kk & 1], kf[kk], s);
      if (kk + 2 < kKs) a[kk & 1] = row_op(q, h, kk + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 pw[2];
    float p[16];
    probs(s, sb, h, qs0, masked, p);
#pragma unroll
    for (int e = 0; e < 8; ++e) pw[e >> 2][e & 3] = E::pack2(p[2 * e], p[2 * e + 1]);
    __builtin_amdgcn_sched_barrier(0);
    vec8 b[2] = {tr_opO(o, h, 0, 0), tr_opO(o, h, 0, 1 % kDBO)};
#pragma unroll
    for (int i = 0; i < 2 * kDBO; ++i) {
      const int tt = i / kDBO, db = i % kDBO;
      acc[db] = E::mfma(b[i & 1], __builtin_bit_cast(vec8, pw[tt]), acc[db]);
      if (i + 2 < 2 * kDBO) b[i & 1] = tr_opO(o, h, (i + 2) / kDBO, (i + 2) % kDBO);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ __forceinline__ void half_k(const uint8_t* sb, int h, int qs0, bool masked) {
    const uint8_t* q = sb + Ld::kQ;
    const uint8_t* o = sb + Ld::kDO;
    f32x16 s = f32x16{}, dp = f32x16{};
    constexpr int kN = kKs + kKsO;
    auto op = [&](int i) { return is_dp(i) ? row_opO(o, h, kstep(i)) : row_op(q, h, kstep(i)); };
    vec8 a[2] = {op(0), op(1)};
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (is_dp(i))
        dp = E::mfma(a[i & 1], vf[kstep(i)], dp);
      else
        s = E::mfma(a[i & 1], kf[kstep(i)], s);
      if (i + 2 < kN) a[i & 1] = op(i + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 sw[2];
    float p[16];
    probs(s, sb, h, qs0, masked, p);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 2 * e;
      const f32x2 dd = pair_vals(sb, Ld::kD, h, r);
      sw[e >> 2][e & 3] = E::pack2(p[r] * (dp[r] - dd[0]), p[r + 1] * (dp[r + 1] - dd[1]));
    }
    __builtin_amdgcn_sched_barrier(0);
    vec8 b[2] = {tr_op(q, h, 0, 0), tr_op(q, h, 0, 1 % kDB)};
#pragma unroll
    for (int i = 0; i < 2 * kDB; ++i) {
      const int tt = i / kDB, db = i % kDB;
      acc[db] = E::mfma(b[i & 1], __builtin_bit_cast(vec8, sw[tt]), acc[db]);
      if (i + 2 < 2 * kDB) b[i & 1] = tr_op(q, h, (i + 2) / kDB, (i + 2) % kDB);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Block-sparse dK/dV: a key block that many query tiles see (a global block
// of the mask) would leave one workgroup walking all of them.  Its list is
// cut into up to kSplit chunks of at least kChunk tiles, each run by its own
// workgroup, which writes fp32 partial dK^T and dV^T to the workspace; the
// last of them to finish (a per-key-block counter, zeroed by the dQ kernel)
// adds the partials in chunk order, so the result stays deterministic.
constexpr int kSplit = kBwdSparseSplit, kChunk = 32;
struct SplitArgs {
  int* cnt;        // [B*H][key blocks of kRes], zeroed by bwd_dq each call
  float* part_dv;  // [kSplit][B*H][N][d_v]
  float* part_dk;  // [kSplit][B*H][N][d]
};
// Byte offsets of those arrays in the block-sparse workspace, after the
// fp32 D and -LSE log2(e) of every query.
struct SparseWs {
  size_t cnt, part_dv, part_dk, bytes;
  SparseWs(int64_t bh, int64_t n, int64_t d, int64_t dv) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    cnt = up((size_t)(8 * bh * n));
    part_dv = up(cnt + (size_t)(4 * bh * ((n + kRes - 1) / kRes)));
    part_dk = part_dv + (size_t)(4 * kSplit * bh * n * dv);
    bytes = part_dk + (size_t)(4 * kSplit * bh * n * d);
  }
};

// One lane's column of a transposed fp32 accumulator as row `row` of a dense
// [.][D] fp32 array, and the sum of such rows over the first n slots.
template <int D, int NA>
__device__ __forceinline__ void store_row_f32(float* base, int row, int g, const f32x16 (&acc)[NA]) {
  float* orow = base + (int64_t)row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * gq + 4 * g) =
          f32x4{acc[db][4 * gq], acc[db][4 * gq + 1], acc[db][4 * gq + 2], acc[db][4 * gq + 3]};
}
template <int D, int NA>
__device__ __forceinline__ void sum_rows_f32(const float* base, int64_t slot, int n, int row, int g,
                                             f32x16 (&acc)[NA]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  for (int z = 0; z < n; ++z) {
    const float* orow = base + z * slot + (int64_t)row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(orow + db * 32 + 8 * gq + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[db][4 * gq + j] += v[j];
      }
  }
}

// Workgroups per CU: two below d = 256; with a 256-wide side one, so that each wave
// may hold 512 registers (its resident operands alone take 128).
template <int D, int DV = D> constexpr int kBwdOcc = (D > 128 || DV > 128) ? 1 : 2;

template <bool IsBf16, int D, bool Causal, int Mode, int DV>
__global__ __launch_bounds__(kThr, (kBwdOcc<D, DV>)) void bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ NLse, const float* __restrict__ Dsum,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int win, int H, int BH, float c,
    float dk_mul, uint32_t k_sign, Layout in, Layout out, Layout lv, Layout outv,
    const uint8_t* __restrict__ bmask, int64_t m_sb, int64_t m_sh, SplitArgs split) {
  using T = STile<D>;
  using TO = STile<DV>;
  using Ld = DkdvLds<D, DV>;
  constexpr bool kSparse = Mode == kModeSparse;
  if constexpr (DV == D) lv = in, outv = out;  // one layout: the d_v addressing folds away
  static_assert(kT == kSparseBlock && kRes % kSparseBlock == 0, "mask blocks are tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Ld::kBytes + (kSparse ? kSparseBytes : 0)];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x % BH;
  // heaviest (earliest keys) first; block-sparse: the chunks of a key block together
  const int kblk = kSparse ? blockIdx.x / BH / kSplit : blockIdx.x / BH;
  const int z = kSparse ? blockIdx.x / BH % kSplit : 0;
  const int b = bh / H, h = bh - b * H;
  const int64_t head = b * in.sb + h * in.sh, head_out = b * out.sb + h * out.sh;
  const int64_t head_v = b * lv.sb + h * lv.sh, head_dv = b * outv.sb + h * outv.sh;
  const int k0 = kblk * kRes, kw0 = k0 + 32 * wave;

  constexpr bool kWin = Causal && Mode == kModeWindow;
  DkdvBlock<IsBf16, D, Causal, Mode, DV> blk;
  blk.init(lane, N, win, kw0, c);
  load_resident<IsBf16, D>(blk.kf, K + head, N, blk.my_k, in.sn, blk.g, k_sign);
  // V^T is used only in pass K; at d = 256 it is loaded there, which keeps
  // its 64 registers free during pass V
  constexpr bool kLateV = D > 128;
  if constexpr (!kLateV) load_resident<IsBf16, DV>(blk.vf, V + head_v, N, blk.my_k, lv.sn, blk.g, 0u);

  // query tiles that can see these keys: from the diagonal to the end of the
  // last key's sliding window
  const int n_tiles = kWin ? min((N + kT - 1) / kT, (k0 + kRes - 1 + win - 1) / kT + 1)
                           : (N + kT - 1) / kT;
  const int t_first = Causal ? k0 / kT : 0;  // earlier query tiles see none of these keys
  // Block-sparse: the query tiles some key block of this workgroup may be
  // seen by, listed in LDS with one bit per 64-key block; a wave skips the
  // tiles its own key block is hidden from.
  uint32_t* const list = reinterpret_cast<uint32_t*>(smem + Ld::kBytes);
  int n_it = n_tiles - t_first;
  if constexpr (kSparse) {
    const int nb = (N + kT - 1) / kT, kb0 = k0 / kSparseBlock;
    const uint8_t* m = bmask + (bh / H) * m_sb + (bh % H) * m_sh;
    n_it = compact_tiles<kW>(list, n_tiles, [&](int it) {
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < kRes / kSparseBlock; ++i) {
        const int kb = kb0 + i;
        if (it >= t_first && kb < nb && (!Causal || kb <= it) && m[(int64_t)it * nb + kb] != 0)
          bits |= 1u << i;
      }
      return bits;
    });
  }
  // query tile at position i, and whether this wave's keys may be seen from it
  auto tile_of = [&](int i) {
    if constexpr (kSparse) return i < n_it ? __builtin_amdgcn_readfirstlane((int)(list[i] & 0xFFFFu)) : n_tiles;
    else return t_first + i;
  };
  auto wave_sees = [&](int i) {
    if constexpr (kSparse) return ((list[i] >> (16 + wave / 2)) & 1u) != 0;
    else return true;
  };
  const uint16_t* q_h = Q + head;
  const uint16_t* do_h = dO + head_v;
  const float* nl_h = NLse + (int64_t)bh * N;
  const float* d_h = Dsum + (int64_t)bh * N;
  uint32_t src[T::kPerWave], srcO[TO::kPerWave];
  T::sources(wave, lane, (uint32_t)(2 * in.sn), src);
  TO::sources(wave, lane, (uint32_t)(2 * lv.sn), srcO);
  const uint32_t lds0 = lds_u32(smem);

  // the copies of query tile it into stage st (-LSE2 by wave 0, D by wave 1)
  auto issue = [&](int it, int st) {
    const int qt0 = it * kT;
    const uint32_t base = lds0 + (uint32_t)(st * Ld::kStage);
    copy_tile<D>(base + Ld::kQ, q_h, N, qt0, in.sn, wave, src);
    copy_tile<DV>(base + Ld::kDO, do_h, N, qt0, lv.sn, wave, srcO);
    const int left = N - qt0;
    if (wave < 2) {
      const i32x4 rs = make_rsrc(wave == 0 ? nl_h + qt0 : d_h + qt0, left > 0 ? (uint32_t)left * 4u : 0u);
      dma4(rs, base + (uint32_t)(wave == 0 ? Ld::kLse : Ld::kD), (uint32_t)lane * 4u);
    }
  };
  // wave-uniform: does tile it reach this wave's keys, and can it need a mask?
  auto live = [&](int it) {
    return kw0 < N && !(Causal && it * kT + kT - 1 < kw0) && !(kWin && it * kT > kw0 + 31 + win - 1);
  };
  auto masked = [&](int it) {
    const int qt0 = it * kT;
    return (Causal && qt0 < kw0 + 32) || (kWin && qt0 + kT - 1 >= kw0 + win) || qt0 + kT > N ||
           kw0 + 32 > N;
  };

  // list positions [i0, i1) of this workgroup (block-sparse chunks)
  int i0 = 0, i1 = n_it, n_chunks = 1;
  if constexpr (kSparse) {
    n_chunks = min(kSplit, max(1, n_it / kChunk));
    if (z >= n_chunks) return;  // workgroup-uniform
    const int per = (n_it + n_chunks - 1) / n_chunks;
    i0 = z * per;
    i1 = min(n_it, i0 + per);
  }
  const int n_mine = i1 - i0;

  issue(tile_of(i0), 0);
  wait_copies();
  __syncthreads();
  // ---- pass V
  blk.zero();
  for (int i = i0; i < i1; ++i) {
    const int it = tile_of(i), st = (i - i0) & 1;
    // the next tile, or (after the last one) the first tile again for pass K
    issue(tile_of(i + 1 < i1 ? i + 1 : i0), st ^ 1);
    if (live(it) && wave_sees(i)) {
      const uint8_t* sb = smem + st * Ld::kStage;
      const bool m = masked(it);
#pragma unroll
      for (int h = 0; h < 2; ++h) blk.half_v(sb, h, it * kT + 32 * h, m);
    }
    wait_copies();
    __syncthreads();
  }
  const bool store = kw0 < N && blk.my_k < N;
  const int64_t slot_v = (int64_t)BH * N * DV, slot_k = (int64_t)BH * N * D;
  if (kSparse && n_chunks > 1) {
    if (store) store_row_f32<DV>(split.part_dv + z * slot_v + (int64_t)bh * N * DV, blk.my_k, blk.g, blk.acc);
  } else if (store) {
    store_row<IsBf16, DV>(dV + head_dv, blk.my_k, outv.sn, blk.g, blk.acc, 1.f);
  }
  if constexpr (kLateV) load_resident<IsBf16, DV>(blk.vf, V + head_v, N, blk.my_k, lv.sn, blk.g, 0u);
  // ---- pass K; the first tile is already in stage n_mine & 1
  blk.zero();
  for (int i = i0; i < i1; ++i) {
    const int it = tile_of(i), st = (i - i0 + n_mine) & 1;
    if (i + 1 < i1) issue(tile_of(i + 1), st ^ 1);
    if (live(it) && wave_sees(i)) {
      const uint8_t* sb = smem + st * Ld::kStage;
      const bool m = masked(it);
#pragma unroll
      for (int h = 0; h < 2; ++h) blk.half_k(sb, h, it * kT + 32 * h, m);
    }
    wait_copies();
    __syncthreads();
  }
  if (kSparse && n_chunks > 1) {
    if (store) store_row_f32<D>(split.part_dk + z * slot_k + (int64_t)bh * N * D, blk.my_k, blk.g, blk.acc);
    // the last chunk to finish adds the partials in chunk order
    __threadfence();
    __syncthreads();
    int* flag = reinterpret_cast<int*>(smem);  // the stages are free: no copy is in flight
    if (threadIdx.x == 0) flag[0] = atomicAdd(split.cnt + (int64_t)bh * ((N + kRes - 1) / kRes) + kblk, 1);
    __syncthreads();
    if (flag[0] != n_chunks - 1) return;
    __threadfence();
    if (!store) return;
    sum_rows_f32<DV>(split.part_dv + (int64_t)bh * N * DV, slot_v, n_chunks, blk.my_k, blk.g, blk.acc);
    store_row<IsBf16, DV>(dV + head_dv, blk.my_k, outv.sn, blk.g, blk.acc, 1.f);
    sum_rows_f32<D>(split.part_dk + (int64_t)bh * N * D, slot_k, n_chunks, blk.my_k, blk.g, blk.acc);
    store_row<IsBf16, D>(dK + head_out, blk.my_k, out.sn, blk.g, blk.acc, dk_mul);
    return;
  }
  if (store) store_row<IsBf16, D>(dK + head_out, blk.my_k, out.sn, blk.g, blk.acc, dk_mul);
}

// ---------------------------------------------------------------- dK, dV (wave pairs)
// Plain and sliding-window masks, d = d_v <= 128.  A workgroup of 8 waves
// keeps 128 keys resident; waves w and w + 4 (one SIMD) share keys
// kw0 .. kw0 + 31 and split the work on each streamed 64-query tile:
//   wave A (w < 4): S = Q K^T, P = exp2(c S - LSE2), P to LDS;  dV^T += dO^T P
//   wave B (w >= 4):  dP = dO V^T;  P from LDS, dS = P (dP - D); dK^T += Q^T dS
// In the first phase of a tile A forms the scores and probabilities while B
// forms dP; a workgroup barrier hands P over; in the second phase A
// accumulates dV while B forms dS and accumulates dK.  S is formed once per
// (query, key) pair instead of once in each of two passes, and the Q and dO
// tiles stream through LDS once.  The arithmetic of every result is that of
// the two-pass kernel above (same MFMA chains, same fp32 P and dS formulas),
// so the gradients are bitwise the same.
constexpr int kPW = 8;            // waves of the pair kernel
constexpr int kPThr = 64 * kPW;

template <int D> struct PairLds {
  using St = DkdvLds<D, D>;
  static constexpr int kStage = St::kStage;          // Q, dO, -LSE log2(e), D of 64 queries
  static constexpr int kP = 2 * kStage;              // P of [pair][half]: 16 fp32 a lane
  static constexpr int kPHalf = 64 * 16 * 4;         // 4 KB
  static constexpr int kBytes = kP + 4 * 2 * kPHalf;
  static_assert(kBytes <= 160 * 1024, "fits the LDS of a CU");
};

// This wave's copies of a 64-row streamed tile when 8 waves share them:
// copy i of wave w fills LDS bytes [(w + 8 i) KB, +1 KB).
template <int D> struct PairCopy {
  using T = STile<D>;
  static constexpr int kPerWave = T::kCopies / kPW;
  static_assert(kPerWave * kPW == T::kCopies, "tile copies split evenly over 8 waves");
  static __device__ __forceinline__ void sources(int wave, int lane, uint32_t row_bytes,
                                                 uint32_t (&src)[kPerWave]) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int byte = (wave + kPW * i) * 1024 + 16 * lane;
      const int r = byte / T::kRowBytes, phys = (byte % T::kRowBytes) / 16;
      src[i] = (uint32_t)tile_row(r) * row_bytes + (uint32_t)(16 * (phys ^ T::swz(r)));
    }
  }
  static __device__ __forceinline__ void copy(uint32_t lds_addr, const uint16_t* base, int rows, int row0,
                                              int64_t sn, int wave, const uint32_t (&src)[kPerWave]) {
    const int left = rows - row0;
    const i32x4 rs = make_rsrc(base + (int64_t)row0 * sn,
                               left > 0 ? (uint32_t)(left - 1) * (uint32_t)(2 * sn) + (uint32_t)T::kDataBytes : 0u);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) dma16(rs, lds_addr + (uint32_t)((wave + kPW * i) * 1024), src[i]);
  }
};

// Workgroup barrier that waits for this wave's LDS traffic only (the HBM ->
// LDS copies in flight keep going; they are waited for at the end of a tile).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool IsBf16, int D, bool Causal, int Mode>
__global__ __launch_bounds__(kPThr, 1) void bwd_dkdv_pair(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ NLse, const float* __restrict__ Dsum,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int win, int H, int BH, float c,
    float dk_mul, uint32_t k_sign, Layout in, Layout out) {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using Ld = PairLds<D>;
  using St = DkdvLds<D, D>;
  using PC = PairCopy<D>;
  static_assert(Mode == kModePlain || Mode == kModeWindow, "plain and window masks");
  constexpr bool kWin = Causal && Mode == kModeWindow;
  constexpr int kKs = D / 16, kDB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Ld::kBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave & 3;
  const bool role_a = wave < 4;  // wave-uniform
  const int bh = blockIdx.x % BH;
  const int kblk = blockIdx.x / BH;  // heaviest (earliest keys) first
  const int b = bh / H, h = bh - b * H;
  const int64_t head = b * in.sb + h * in.sh, head_out = b * out.sb + h * out.sh;
  const int k0 = kblk * kRes, kw0 = k0 + 32 * pair;

  DkdvBlock<IsBf16, D, Causal, Mode, D> blk;
  blk.init(lane, N, win, kw0, c);

  const int n_tiles = kWin ? min((N + kT - 1) / kT, (k0 + kRes - 1 + win - 1) / kT + 1) : (N + kT - 1) / kT;
  const int t_first = Causal ? k0 / kT : 0;
  const int n_it = n_tiles - t_first;
  const uint16_t* q_h = Q + head;
  const uint16_t* do_h = dO + head;
  const float* nl_h = NLse + (int64_t)bh * N;
  const float* d_h = Dsum + (int64_t)bh * N;
  uint32_t src[PC::kPerWave];
  PC::sources(wave, lane, (uint32_t)(2 * in.sn), src);
  const uint32_t lds0 = lds_u32(smem);

  auto issue = [&](int it, int st) {
    const int qt0 = it * kT;
    const uint32_t base = lds0 + (uint32_t)(st * Ld::kStage);
    PC::copy(base + St::kQ, q_h, N, qt0, in.sn, wave, src);
    PC::copy(base + St::kDO, do_h, N, qt0, in.sn, wave, src);
    const int left = N - qt0;
    if (wave < 2) {
      const i32x4 rs = make_rsrc(wave == 0 ? nl_h + qt0 : d_h + qt0, left > 0 ? (uint32_t)left * 4u : 0u);
      dma4(rs, base + (uint32_t)(wave == 0 ? St::kLse : St::kD), (uint32_t)lane * 4u);
    }
  };
  auto live = [&](int it) {
    return kw0 < N && !(Causal && it * kT + kT - 1 < kw0) && !(kWin && it * kT > kw0 + 31 + win - 1);
  };
  auto masked = [&](int it) {
    const int qt0 = it * kT;
    return (Causal && qt0 < kw0 + 32) || (kWin && qt0 + kT - 1 >= kw0 + win) || qt0 + kT > N ||
           kw0 + 32 > N;
  };
  // P of (this pair, half hh): 16 fp32 a lane as four 16-byte chunks, chunk j
  // of lane l at 16 (64 j + l) (each chunk write / read is 1 KB contiguous)
  float* const pbuf = reinterpret_cast<float*>(smem + Ld::kP + pair * 2 * Ld::kPHalf);
  auto p_at = [&](int hh, int j) { return reinterpret_cast<f32x4*>(pbuf + hh * (Ld::kPHalf / 4)) + 64 * j + lane; };

  issue(t_first, 0);
  wait_copies();
  __syncthreads();
  blk.zero();
  if (role_a) {
    load_resident<IsBf16, D>(blk.kf, K + head, N, blk.my_k, in.sn, blk.g, k_sign);
    for (int i = 0; i < n_it; ++i) {
      const int it = t_first + i, st = i & 1;
      if (i + 1 < n_it) issue(it + 1, st ^ 1);
      const uint8_t* sb = smem + st * Ld::kStage;
      const bool lv = live(it);
      u32x4 pw[2][2];
      if (lv) {
        const bool m = masked(it);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint8_t* q = sb + St::kQ;
          f32x16 s = f32x16{};
          vec8 a[2] = {blk.row_op(q, hh, 0), blk.row_op(q, hh, 1)};
#pragma unroll
          for (int kk = 0; kk < kKs; ++kk) {
            s = E::mfma(a[kk & 1], blk.kf[kk], s);
            if (kk + 2 < kKs) a[kk & 1] = blk.row_op(q, hh, kk + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
          float p[16];
          blk.probs(s, sb, hh, it * kT + 32 * hh, m, p);
#pragma unroll
          for (int e = 0; e < 8; ++e) pw[hh][e >> 2][e & 3] = E::pack2(p[2 * e], p[2 * e + 1]);
#pragma unroll
          for (int j = 0; j < 4; ++j) *p_at(hh, j) = f32x4{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
        }
      }
      lds_barrier();  // P handed to wave B
      if (lv) {
        const uint8_t* o = sb + St::kDO;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          vec8 bq[2] = {blk.tr_op(o, hh, 0, 0), blk.tr_op(o, hh, 0, 1 % kDB)};
#pragma unroll
          for (int i2 = 0; i2 < 2 * kDB; ++i2) {
            const int tt = i2 / kDB, db = i2 % kDB;
            blk.acc[db] = E::mfma(bq[i2 & 1], __builtin_bit_cast(vec8, pw[hh][tt]), blk.acc[db]);
            if (i2 + 2 < 2 * kDB) bq[i2 & 1] = blk.tr_op(o, hh, (i2 + 2) / kDB, (i2 + 2) % kDB);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      wait_copies();
      __syncthreads();
    }
    if (kw0 < N && blk.my_k < N) store_row<IsBf16, D>(dV + head_out, blk.my_k, out.sn, blk.g, blk.acc, 1.f);
  } else {
    load_resident<IsBf16, D>(blk.vf, V + head, N, blk.my_k, in.sn, blk.g, 0u);
    for (int i = 0; i < n_it; ++i) {
      const int it = t_first + i, st = i & 1;
      if (i + 1 < n_it) issue(it + 1, st ^ 1);
      const uint8_t* sb = smem + st * Ld::kStage;
      const bool lv = live(it);
      f32x16 dp[2];
      if (lv) {
        const uint8_t* o = sb + St::kDO;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          dp[hh] = f32x16{};
          vec8 a[2] = {blk.row_opO(o, hh, 0), blk.row_opO(o, hh, 1)};
#pragma unroll
          for (int kk = 0; kk < kKs; ++kk) {
            dp[hh] = E::mfma(a[kk & 1], blk.vf[kk], dp[hh]);
            if (kk + 2 < kKs) a[kk & 1] = blk.row_opO(o, hh, kk + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      lds_barrier();  // P from wave A
      if (lv) {
        const uint8_t* q = sb + St::kQ;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float p[16];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 v4 = *p_at(hh, j);
            p[4 * j] = v4[0], p[4 * j + 1] = v4[1], p[4 * j + 2] = v4[2], p[4 * j + 3] = v4[3];
          }
          u32x4 sw[2];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 2 * e;
            const f32x2 dd = blk.pair_vals(sb, St::kD, hh, r);
            sw[e >> 2][e & 3] = E::pack2(p[r] * (dp[hh][r] - dd[0]), p[r + 1] * (dp[hh][r + 1] - dd[1]));
          }
          __builtin_amdgcn_sched_barrier(0);
          vec8 bq[2] = {blk.tr_op(q, hh, 0, 0), blk.tr_op(q, hh, 0, 1 % kDB)};
#pragma unroll
          for (int i2 = 0; i2 < 2 * kDB; ++i2) {
            const int tt = i2 / kDB, db = i2 % kDB;
            blk.acc[db] = E::mfma(bq[i2 & 1], __builtin_bit_cast(vec8, sw[tt]), blk.acc[db]);
            if (i2 + 2 < 2 * kDB) bq[i2 & 1] = blk.tr_op(q, hh, (i2 + 2) / kDB, (i2 + 2) % kDB);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      wait_copies();
      __syncthreads();
    }
    if (kw0 < N && blk.my_k < N) store_row<IsBf16, D>(dK + head_out, blk.my_k, out.sn, blk.g, blk.acc, dk_mul);
  }
}

// ---------------------------------------------------------------- D and dQ
// Per wave: 32 resident queries (lane column = query).  Key tiles of 64 rows
// (K, V) stream through two LDS stages, twice.  For each 32-key half:
//   S^T = K Q^T and dP^T = V dO^T (A = K / V rows from LDS, B = Q^T / dO^T resident)
//   P^T = exp2(c S^T - LSE2)                           (LSE2: lane scalar)
//   pass 1:  D += sum over the keys of P^T dP^T
//   pass 2:  dS^T = P^T (dP^T - D),  dQ^T += K^T dS^T  (A = K^T by transpose reads)
template <int D, int DV = D> struct DqLds {
  static constexpr int kK = 0;
  static constexpr int kV = STile<D>::kBytes;                 // V rows of d_v
  static constexpr int kStage = kV + STile<DV>::kBytes;
  static constexpr int kBytes = 2 * kStage;
};

template <bool IsBf16, int D, bool Causal, int Mode, int DV>
__global__ __launch_bounds__(kThr, (kBwdOcc<D, DV>)) void bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ Dsum,
    float* __restrict__ NLse, uint16_t* __restrict__ dQ, int N, int win, int H, int BH, int n_qblocks,
    float c, float dq_mul, uint32_t q_sign, Layout in, Layout out, Layout lv,
    const uint8_t* __restrict__ bmask, int64_t m_sb, int64_t m_sh, SplitArgs split) {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using T = STile<D>;
  using TO = STile<DV>;
  using Ld = DqLds<D, DV>;
  constexpr int kKs = D / 16, kDB = D / 32, kKsO = DV / 16;
  if constexpr (DV == D) lv = in;  // one layout: the d_v addressing folds away
  constexpr bool kSparse = Mode == kModeSparse;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Ld::kBytes + (kSparse ? kSparseBytes : 0)];

  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (Causal) qb = n_qblocks - 1 - qb;  // heaviest first
  const int b = bh / H, h = bh - b * H;
  const int64_t head = b * in.sb + h * in.sh, head_v = b * lv.sb + h * lv.sh;
  if constexpr (kSparse) {
    // the dK/dV kernel's per-key-block chunk counters of this head start at zero
    if (qb == 0)
      for (int i = threadIdx.x; i < n_qblocks; i += kThr) split.cnt[(int64_t)bh * n_qblocks + i] = 0;
  }
  const int q0 = qb * kRes, qw0 = q0 + 32 * wave, my_q = qw0 + l32;

  vec8 qf[kKs], of[kKsO];
  load_resident<IsBf16, D>(qf, Q + head, N, my_q, in.sn, g, q_sign);
  load_resident<IsBf16, DV>(of, dO + head_v, N, my_q, lv.sn, g, 0u);
  const bool q_ok = my_q < N;
  const float lse2 = q_ok ? LSE[(int64_t)bh * N + my_q] * 1.4426950408889634f : INFINITY;

  const int last_row = min(N, q0 + kRes) - 1;
  const int n_tiles = Causal ? last_row / kT + 1 : (N + kT - 1) / kT;
  // first key tile any query of the block can see (sliding window)
  constexpr bool kWin = Causal && Mode == kModeWindow;
  const int t_lo = kWin ? max(0, q0 - win + 1) / kT : 0;
  // Block-sparse: the key tiles some query block of this workgroup may see,
  // listed in LDS with one bit per 64-row query block; a wave skips the tiles
  // hidden from its own query block.
  uint32_t* const list = reinterpret_cast<uint32_t*>(smem + Ld::kBytes);
  int n_it = n_tiles - t_lo;
  if constexpr (kSparse) {
    const int nb = (N + kT - 1) / kT, qb0 = q0 / kSparseBlock;
    const uint8_t* m = bmask + (bh / H) * m_sb + (bh % H) * m_sh;
    n_it = compact_tiles<kW>(list, n_tiles, [&](int jt) {
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < kRes / kSparseBlock; ++i) {
        const int qbk = qb0 + i;
        if (qbk < nb && (!Causal || jt <= qbk) && m[(int64_t)qbk * nb + jt] != 0) bits |= 1u << i;
      }
      return bits;
    });
  }
  auto tile_of = [&](int i) {
    if constexpr (kSparse) return i < n_it ? __builtin_amdgcn_readfirstlane((int)(list[i] & 0xFFFFu)) : n_tiles;
    else return t_lo + i;
  };
  auto wave_sees = [&](int i) {
    if constexpr (kSparse) return ((list[i] >> (16 + wave / 2)) & 1u) != 0;
    else return true;
  };
  const bool wave_live = qw0 < N;
  const uint16_t* k_h = K + head;
  const uint16_t* v_h = V + head_v;
  uint32_t src[T::kPerWave], srcO[TO::kPerWave];
  T::sources(wave, lane, (uint32_t)(2 * in.sn), src);
  TO::sources(wave, lane, (uint32_t)(2 * lv.sn), srcO);
  const uint32_t lds0 = lds_u32(smem);

  auto issue = [&](int it, int st) {
    const uint32_t base = lds0 + (uint32_t)(st * Ld::kStage);
    copy_tile<D>(base + Ld::kK, k_h, N, it * kT, in.sn, wave, src);
    copy_tile<DV>(base + Ld::kV, v_h, N, it * kT, lv.sn, wave, srcO);
  };

  // Whether key half ks0 .. ks0 + 31 hides some key from some query of this
  // wave (causal diagonal, left edge of the window, end of the sequence); the
  // other halves skip the per-element masks.  Rows past N need none: their
  // LSE is +inf, so their probabilities are 0.
  auto needs_mask = [&](int ks0) {
    return (Causal && ks0 + 31 > qw0) || (kWin && ks0 <= qw0 + 31 - win) || ks0 + 32 > N;
  };
  // S^T and dP^T of key half kh of the tile in stage st, and P^T; register e
  // of lane half g holds key ks0 + 16 (e >> 3) + 8 g + (e & 7).  One code path
  // for both kinds of half, with a wave-uniform branch around the masks, so
  // that the loop holds one copy and no register copies at a join.
  auto scores_at = [&](int st, int kh, int ks0, f32x16& p, f32x16& dp) {
    const uint8_t* k_lds = smem + st * Ld::kStage + Ld::kK;
    const uint8_t* v_lds = smem + st * Ld::kStage + Ld::kV;
    f32x16 s = f32x16{};
    dp = f32x16{};
    const int r = 32 * kh + l32;
#pragma unroll
    for (int kk = 0; kk < (kKs > kKsO ? kKs : kKsO); ++kk) {
      if (kk < kKs) s = E::mfma(row_frag<IsBf16, D>(k_lds, r, g, kk), qf[kk], s);
      if (kk < kKsO) dp = E::mfma(row_frag<IsBf16, DV>(v_lds, r, g, kk), of[kk], dp);
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) p[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], c, -lse2));
    if (needs_mask(ks0)) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int kj = ks0 + 16 * (rr >> 3) + 8 * g + (rr & 7);
        if (kj >= N || (Causal && kj > my_q) || (kWin && kj <= my_q - win)) p[rr] = 0.f;
      }
    }
  };

  // ---- pass 1: D = sum_j P_ij dP_ij
  float dpart = 0.f;
  issue(tile_of(0), 0);
  wait_copies();
  __syncthreads();
  for (int i = 0; i < n_it; ++i) {
    const int it = tile_of(i), st = i & 1;
    // the next tile, or (after the last one) the first tile again for pass 2
    issue(tile_of(i + 1 < n_it ? i + 1 : 0), st ^ 1);
    const int kt0 = it * kT;
    if (wave_live && wave_sees(i)) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int ks0 = kt0 + 32 * kh;
        if ((Causal && ks0 > qw0 + 31) || (kWin && ks0 + 31 <= qw0 - win) || ks0 >= N) continue;
        f32x16 p, dp;
        scores_at(st, kh, ks0, p, dp);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) dpart = __builtin_fmaf(p[rr], dp[rr], dpart);
      }
    }
    wait_copies();
    __syncthreads();
  }
  const float dsum = xhalf_sum(dpart);
  if (wave_live && q_ok && g == 0) {
    Dsum[(int64_t)bh * N + my_q] = dsum;
    NLse[(int64_t)bh * N + my_q] = -lse2;  // read by the dK/dV kernel
  }

  // ---- pass 2: dQ^T += K^T dS^T; the first tile is already in stage n_it & 1
  f32x16 dq[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) dq[i] = f32x16{};
  for (int i = 0; i < n_it; ++i) {
    const int it = tile_of(i), st = (i + n_it) & 1;
    if (i + 1 < n_it) issue(tile_of(i + 1), st ^ 1);
    const int kt0 = it * kT;
    if (wave_live && wave_sees(i)) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int ks0 = kt0 + 32 * kh;
        if ((Causal && ks0 > qw0 + 31) || (kWin && ks0 + 31 <= qw0 - win) || ks0 >= N) continue;
        f32x16 p, dp;
        scores_at(st, kh, ks0, p, dp);
        u32x4 sw[2];
#pragma unroll
        for (int e = 0; e < 16; e += 2)
          sw[e >> 3][(e & 7) >> 1] = E::pack2(p[e] * (dp[e] - dsum), p[e + 1] * (dp[e + 1] - dsum));
        const uint8_t* k_lds = smem + st * Ld::kStage + Ld::kK;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            dq[db] = E::mfma(tr_frag<IsBf16, D>(k_lds, lane, 2 * kh + t, db),
                             __builtin_bit_cast(vec8, sw[t]), dq[db]);
      }
    }
    wait_copies();
    __syncthreads();
  }
  if (!wave_live || !q_ok) return;
  store_row<IsBf16, D>(dQ + (b * out.sb + h * out.sh), my_q, out.sn, g, dq, dq_mul);
}

// ---------------------------------------------------------------- dQ (wave pairs, one pass)
// Plain and sliding-window masks, d = d_v <= 128.  A workgroup of 8 waves
// keeps 128 queries resident; waves w and w + 4 (one SIMD) share queries
// qw0 .. qw0 + 31 and stream the 64-key tiles of K and V once:
//   wave A (w < 4):  S^T = K Q^T, P^T = exp2(c S^T - LSE2), P (fp32) to LDS
//   wave B (w >= 4): dP^T = V dO^T;  P from LDS;  D_i += sum_j P_ij dP_ij;
//                    dQ~^T += K^T (P (dP - D~))^T,  B^T += K^T P^T
// with D~_i = dO_i . O_i from the stored output and B_i = sum_j P_ij k_j.
// Since
//     dQ_i / scale = sum_j P_ij (dP_ij - D_i) k_j
//                  = dQ~_i - (D_i - D~_i) B_i
// (exact), one pass gives dQ with the exact row term D_i = sum_j P_ij dP_ij:
// D~ only keeps the operand P (dP - D~) as small as P (dP - D) (O's rounding
// moves D~ by about 2^-9 relative, and that difference reaches dQ through the
// fp32 correction, not through a bf16 operand).  D is accumulated in the
// order of the two-pass kernel, so the dK/dV kernel that reads it is
// unchanged bit for bit.
//
// Wave B's two K^T products share each transpose read of K, so a 32 x 64
// block costs 48 KB of LDS operand and P traffic against 64 MFMAs.  Wave A
// runs one key tile ahead of wave B: in step i it forms P of tile i while B
// consumes P of tile i - 1, which the barrier ending step i - 1 handed over.
// K tiles sit in a ring of three LDS slots (A reads tile i, B tile i - 1,
// tile i + 1 is in flight), V tiles and P sets in rings of two.
template <int D> struct DqPairLds {
  static constexpr int kTile = STile<D>::kBytes;     // one 64-row tile of K or V
  static constexpr int kK = 0;                       // K ring: tile t in slot t % 3
  static constexpr int kV = 3 * kTile;               // V ring: slot t % 2
  static constexpr int kP = kV + 2 * kTile;          // P ring: set t % 2 of [pair][key half]
  static constexpr int kPHalf = 64 * 16 * 4;         // 4 KB: 16 fp32 a lane
  static constexpr int kPSet = 4 * 2 * kPHalf;
  static constexpr int kBytes = kP + 2 * kPSet;
  static_assert(kBytes <= 160 * 1024, "fits the LDS of a CU");
};

template <bool IsBf16, int D, bool Causal, int Mode>
__global__ __launch_bounds__(kPThr, 1) void bwd_dq_pair(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ Dsum, float* __restrict__ NLse, uint16_t* __restrict__ dQ, int N, int win, int H,
    int BH, int n_qblocks, float c, float dq_mul, uint32_t q_sign, Layout in, Layout out) {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using Ld = DqPairLds<D>;
  using PC = PairCopy<D>;
  using T = STile<D>;
  typedef __attribute__((address_space(3))) const vec8 lds_vec8;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  static_assert(Mode == kModePlain || Mode == kModeWindow, "plain and window masks");
  constexpr bool kWin = Causal && Mode == kModeWindow;
  constexpr int kKs = D / 16, kDB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Ld::kBytes];

  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave & 3;
  const bool role_a = wave < 4;
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (Causal) qb = n_qblocks - 1 - qb;  // heaviest first
  const int b = bh / H, h = bh - b * H;
  const int64_t head = b * in.sb + h * in.sh;
  const int q0 = qb * kRes, qw0 = q0 + 32 * pair, my_q = qw0 + l32;
  const bool q_ok = my_q < N;
  const float lse2 = q_ok ? LSE[(int64_t)bh * N + my_q] * 1.4426950408889634f : INFINITY;

  const int last_row = min(N, q0 + kRes) - 1;
  const int n_tiles = Causal ? last_row / kT + 1 : (N + kT - 1) / kT;
  const int t_lo = kWin ? max(0, q0 - win + 1) / kT : 0;
  const int n_it = n_tiles - t_lo;
  const bool pair_live = qw0 < N;
  const uint16_t* k_h = K + head;
  const uint16_t* v_h = V + head;
  uint32_t src[PC::kPerWave];
  PC::sources(wave, lane, (uint32_t)(2 * in.sn), src);
  const uint32_t lds0 = lds_u32(smem);
  auto issue_k = [&](int i) {
    PC::copy(lds0 + (uint32_t)(Ld::kK + (i % 3) * Ld::kTile), k_h, N, (t_lo + i) * kT, in.sn, wave, src);
  };
  auto issue_v = [&](int i) {
    PC::copy(lds0 + (uint32_t)(Ld::kV + (i & 1) * Ld::kTile), v_h, N, (t_lo + i) * kT, in.sn, wave, src);
  };
  // whether key half ks0 .. ks0 + 31 lies wholly outside what this pair's
  // queries see, and whether it can hide some key from some of them
  auto skip_half = [&](int ks0) {
    return !pair_live || (Causal && ks0 > qw0 + 31) || (kWin && ks0 + 31 <= qw0 - win) || ks0 >= N;
  };
  auto needs_mask = [&](int ks0) {
    return (Causal && ks0 + 31 > qw0) || (kWin && ks0 <= qw0 + 31 - win) || ks0 + 32 > N;
  };
  // LDS addresses are kept per lane and per slot in registers (advanced by a
  // scalar from one step to the next, and hidden from the compiler by an
  // empty asm), so that a key half, k step or P chunk only adds a constant in
  // the instruction's offset field.  Otherwise the compiler keeps every
  // (lane offset + constant) sum of the loop live, which does not fit.
  auto hide = [](uint32_t& a) { asm("" : "+v"(a)); };
  auto row_at = [](uint32_t a) { return *(lds_vec8*)(uintptr_t)a; };
  auto tr_at = [](uint32_t lo, uint32_t hi) {
    const auto l = E::read_tr((const lds_void*)(uintptr_t)lo);
    const auto u = E::read_tr((const lds_void*)(uintptr_t)hi);
    return __builtin_shufflevector(l, u, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // k slot step from tile i to tile i + 1 in the ring of three
  auto k_step = [](int i) { return (uint32_t)(i % 3 == 2 ? -2 * Ld::kTile : Ld::kTile); };
  // P of (set, this pair, key half kh): chunk j of lane l at 16 (64 j + l)
  uint32_t pb = lds0 + (uint32_t)(Ld::kP + pair * 2 * Ld::kPHalf + 16 * lane);  // set 0
  auto p_step = [](int i) { return (uint32_t)(i & 1 ? -Ld::kPSet : Ld::kPSet); };
  // the row operand of k step kk: LDS row l32 (+ 32 in the second key half), chunk 2 kk + g
  auto row_off = [&](int kk) { return (uint32_t)T::at(l32, 2 * kk + g); };

  issue_k(0);
  wait_copies();
  __syncthreads();
  if (role_a) {
    vec8 qf[kKs];
    load_resident<IsBf16, D>(qf, Q + head, N, my_q, in.sn, g, q_sign);
    uint32_t kb[kKs];  // K rows, slot of tile i
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk) kb[kk] = lds0 + (uint32_t)Ld::kK + row_off(kk);
    // step i: P of tile i (step n_it only meets the barrier)
    for (int i = 0; i <= n_it; ++i) {
      if (i + 1 < n_it) issue_k(i + 1);
      if (i < n_it) issue_v(i);
      if (i < n_it) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int ks0 = (t_lo + i) * kT + 32 * kh;
          if (skip_half(ks0)) continue;
          constexpr uint32_t kHalfRows = 32 * T::kRowBytes;
          f32x16 s = f32x16{};
          // operand reads run two MFMAs ahead; the fences keep the compiler
          // from hoisting all of them into registers
          vec8 a[2] = {row_at(kb[0] + kh * kHalfRows), row_at(kb[1] + kh * kHalfRows)};
#pragma unroll
          for (int kk = 0; kk < kKs; ++kk) {
            s = E::mfma(a[kk & 1], qf[kk], s);
            if (kk + 2 < kKs) a[kk & 1] = row_at(kb[kk + 2] + kh * kHalfRows);
            __builtin_amdgcn_sched_barrier(0);
          }
          float p[16];
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) p[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], c, -lse2));
          if (needs_mask(ks0)) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int kj = ks0 + 16 * (rr >> 3) + 8 * g + (rr & 7);
              if (kj >= N || (Causal && kj > my_q) || (kWin && kj <= my_q - win)) p[rr] = 0.f;
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(lds_f32x4*)(uintptr_t)(pb + kh * Ld::kPHalf + 1024 * j) =
                f32x4{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
        }
      }
      const uint32_t ks = k_step(i), ps = p_step(i);
#pragma unroll
      for (int kk = 0; kk < kKs; ++kk) kb[kk] += ks, hide(kb[kk]);
      pb += ps;
      hide(pb);
      wait_copies();
      __syncthreads();
    }
  } else {
    vec8 of[kKs];
    load_resident<IsBf16, D>(of, dO + head, N, my_q, in.sn, g, 0u);
    // D~ = dO . O of this lane's query (its d range, then the other half's)
    float dt = 0.f;
    {
      vec8 oo[kKs];
      load_resident<IsBf16, D>(oo, O + head, N, my_q, in.sn, g, 0u);
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) dt = __builtin_fmaf((float)of[ks][e], (float)oo[ks][e], dt);
    }
    const float dtil = xhalf_sum(dt);
    uint32_t vb[kKs], kt_lo[kDB], kt_hi[kDB];  // V rows and K^T reads, slots of tile i - 1
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk) vb[kk] = lds0 + (uint32_t)Ld::kV + row_off(kk);
    {
      // transpose reads of d block db: logical rows 4 g + s / 4 and 8 more
      // (s = lane % 16), k step t adding 16 rows
      const int grp = lane >> 4, s16 = lane & 15, r0 = 4 * g + (s16 >> 2);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int col = 2 * (16 * (grp & 1) + 4 * (s16 & 3)) + 64 * db;
        kt_lo[db] = lds0 + (uint32_t)(Ld::kK + T::at(r0, col >> 4) + (col & 15));
        kt_hi[db] = lds0 + (uint32_t)(Ld::kK + T::at(r0 + 8, col >> 4) + (col & 15));
      }
    }
    f32x16 dq[kDB], bacc[kDB];
#pragma unroll
    for (int i = 0; i < kDB; ++i) dq[i] = f32x16{}, bacc[i] = f32x16{};
    float dpart = 0.f;
    // step i: the products of tile i - 1 (step 0 only meets the barrier)
    for (int i = 0; i <= n_it; ++i) {
      if (i + 1 < n_it) issue_k(i + 1);
      if (i < n_it) issue_v(i);
      if (i > 0) {
        const int it = i - 1;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int ks0 = (t_lo + it) * kT + 32 * kh;
          if (skip_half(ks0)) continue;
          constexpr uint32_t kHalfRows = 32 * T::kRowBytes, kStepRows = 16 * T::kRowBytes;
          f32x16 dp = f32x16{};
          vec8 a[2] = {row_at(vb[0] + kh * kHalfRows), row_at(vb[1] + kh * kHalfRows)};
#pragma unroll
          for (int kk = 0; kk < kKs; ++kk) {
            dp = E::mfma(a[kk & 1], of[kk], dp);
            if (kk + 2 < kKs) a[kk & 1] = row_at(vb[kk + 2] + kh * kHalfRows);
            __builtin_amdgcn_sched_barrier(0);
          }
          float p[16];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 v4 = *(lds_f32x4*)(uintptr_t)(pb + kh * Ld::kPHalf + 1024 * j);
            p[4 * j] = v4[0], p[4 * j + 1] = v4[1], p[4 * j + 2] = v4[2], p[4 * j + 3] = v4[3];
          }
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) dpart = __builtin_fmaf(p[rr], dp[rr], dpart);
          u32x4 sw[2], pw[2];
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            sw[e >> 3][(e & 7) >> 1] = E::pack2(p[e] * (dp[e] - dtil), p[e + 1] * (dp[e + 1] - dtil));
            pw[e >> 3][(e & 7) >> 1] = E::pack2(p[e], p[e + 1]);
          }
          __builtin_amdgcn_sched_barrier(0);
          // K^T operand i2 = (d block i2 / 2, k step 2 kh + i2 % 2) feeds dQ~ and B
          auto kt_op = [&](int t, int db) {
            const uint32_t o = (2 * kh + t) * kStepRows;
            return tr_at(kt_lo[db] + o, kt_hi[db] + o);
          };
          vec8 kt[2] = {kt_op(0, 0), kt_op(1, 0)};
#pragma unroll
          for (int i2 = 0; i2 < 2 * kDB; ++i2) {
            const int db = i2 >> 1, t = i2 & 1;
            dq[db] = E::mfma(kt[t], __builtin_bit_cast(vec8, sw[t]), dq[db]);
            bacc[db] = E::mfma(kt[t], __builtin_bit_cast(vec8, pw[t]), bacc[db]);
            if (i2 + 2 < 2 * kDB) kt[t] = kt_op(t, db + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // slots of tile i
        const uint32_t ks = k_step(it), vs = (uint32_t)(it & 1 ? -Ld::kTile : Ld::kTile);
#pragma unroll
        for (int kk = 0; kk < kKs; ++kk) vb[kk] += vs, hide(vb[kk]);
#pragma unroll
        for (int db = 0; db < kDB; ++db) kt_lo[db] += ks, kt_hi[db] += ks, hide(kt_lo[db]), hide(kt_hi[db]);
        pb += p_step(it);
        hide(pb);
      }
      wait_copies();
      __syncthreads();
    }
    const float dsum = xhalf_sum(dpart);
    if (!pair_live || !q_ok) return;
    if (g == 0) {
      Dsum[(int64_t)bh * N + my_q] = dsum;
      NLse[(int64_t)bh * N + my_q] = -lse2;  // read by the dK/dV kernel
    }
    const float delta = dsum - dtil;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[db][r] = __builtin_fmaf(-delta, bacc[db][r], dq[db][r]);
    store_row<IsBf16, D>(dQ + (b * out.sb + h * out.sh), my_q, out.sn, g, dq, dq_mul);
  }
}

template <bool IsBf16, int D, bool Causal, int Mode, int DV = D>
hipError_t launch(const BwdArgs& a, hipStream_t st) {
  const int N = (int)a.N;
  const int BH = (int)(a.B * a.H);
  const int nblk = (N + kRes - 1) / kRes;
  // |scale| * log2(e); a zero scale is run as the limit scale -> 0+
  const float c = a.scale != 0.f ? __builtin_fabsf(a.scale) * 1.4426950408889634f : 1e-30f;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const int win = (int)(a.window < a.N ? a.window : a.N);  // sliding window (N: plain causal)
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const auto* dout = static_cast<const uint16_t*>(a.dout);
  // workspace: D, then -LSE * log2(e), one fp32 per query each; block-sparse
  // also the chunk counters and partial sums
  float* dsum = static_cast<float*>(a.workspace);
  float* nlse = dsum + a.B * a.H * a.N;
  SplitArgs split{nullptr, nullptr, nullptr};
  if constexpr (Mode == kModeSparse) {
    const SparseWs w(a.B * a.H, a.N, D, DV);
    char* base = static_cast<char*>(a.workspace);
    split = SplitArgs{reinterpret_cast<int*>(base + w.cnt), reinterpret_cast<float*>(base + w.part_dv),
                      reinterpret_cast<float*>(base + w.part_dk)};
  }
  const int kgrid = Mode == kModeSparse ? nblk * BH * kSplit : nblk * BH;
  // dQ (and D into the workspace) first; dK, dV read D afterwards on the same stream
  if constexpr (DV == D && D <= 128 && Mode != kModeSparse) {
    hipLaunchKernelGGL((bwd_dq_pair<IsBf16, D, Causal, Mode>), dim3((unsigned)(nblk * BH)), dim3(kPThr), 0, st,
                       q, k, v, static_cast<const uint16_t*>(a.o), dout, a.lse, dsum, nlse,
                       static_cast<uint16_t*>(a.dq), N, win, (int)a.H, BH, nblk, c, a.scale, q_sign, a.in,
                       a.out);
  } else {
    hipLaunchKernelGGL((bwd_dq<IsBf16, D, Causal, Mode, DV>), dim3((unsigned)(nblk * BH)), dim3(kThr), 0, st,
                       q, k, v, dout, a.lse, dsum, nlse, static_cast<uint16_t*>(a.dq), N, win, (int)a.H,
                       BH, nblk, c, a.scale, q_sign, a.in, a.out, a.lv, a.block_mask, a.mask_sb, a.mask_sh,
                       split);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dK = scale dS^T Q; a negative scale flips the resident K instead of Q
  if constexpr (DV == D && D <= 128 && Mode != kModeSparse) {
    hipLaunchKernelGGL((bwd_dkdv_pair<IsBf16, D, Causal, Mode>), dim3((unsigned)(nblk * BH)), dim3(kPThr), 0,
                       st, q, k, v, dout, nlse, dsum, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv), N, win, (int)a.H, BH, c, a.scale, q_sign, a.in, a.out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bwd_dkdv<IsBf16, D, Causal, Mode, DV>), dim3((unsigned)kgrid), dim3(kThr), 0, st,
                     q, k, v, dout, nlse, dsum, static_cast<uint16_t*>(a.dk),
                     static_cast<uint16_t*>(a.dv), N, win, (int)a.H, BH, c, a.scale, q_sign, a.in, a.out,
                     a.lv, a.outv, a.block_mask, a.mask_sb, a.mask_sh, split);
  return hipGetLastError();
}

// A causal window narrower than N runs the Window instantiations; plain causal
// and unmasked calls run code with no window arithmetic.
template <bool IsBf16, int D>
hipError_t dispatch_d(const BwdArgs& a, hipStream_t s) {
  if (a.block_mask != nullptr)
    return a.causal ? launch<IsBf16, D, true, kModeSparse>(a, s) : launch<IsBf16, D, false, kModeSparse>(a, s);
  if (!a.causal) return launch<IsBf16, D, false, kModePlain>(a, s);
  if (a.window < a.N) return launch<IsBf16, D, true, kModeWindow>(a, s);
  return launch<IsBf16, D, true, kModePlain>(a, s);
}

template <bool IsBf16, int D, int DV>
hipError_t launch_dv(const BwdArgs& a, hipStream_t s) {
  return a.causal ? launch<IsBf16, D, true, kModePlain, DV>(a, s) : launch<IsBf16, D, false, kModePlain, DV>(a, s);
}

template <bool IsBf16>
hipError_t dispatch(const BwdArgs& a, hipStream_t s) {
  // d_v != d (plain masks only): q, k, dq, dk rows of d, v, o, dout, dv rows
  // of d_v; d, d_v in {64, 96, 128, 256}
  if (a.dvw != a.d) {
    if (a.dvw == 256)
      return a.d == 64 ? launch_dv<IsBf16, 64, 256>(a, s)
           : a.d == 96 ? launch_dv<IsBf16, 96, 256>(a, s) : launch_dv<IsBf16, 128, 256>(a, s);
    if (a.d == 256)
      return a.dvw == 64 ? launch_dv<IsBf16, 256, 64>(a, s)
           : a.dvw == 96 ? launch_dv<IsBf16, 256, 96>(a, s) : launch_dv<IsBf16, 256, 128>(a, s);
    if (a.d == 128) return a.dvw == 64 ? launch_dv<IsBf16, 128, 64>(a, s) : launch_dv<IsBf16, 128, 96>(a, s);
    if (a.d == 96) return a.dvw == 64 ? launch_dv<IsBf16, 96, 64>(a, s) : launch_dv<IsBf16, 96, 128>(a, s);
    return a.dvw == 96 ? launch_dv<IsBf16, 64, 96>(a, s) : launch_dv<IsBf16, 64, 128>(a, s);
  }
  if (a.d == 256) {  // plain masks, the sliding window and block masks
    if (a.block_mask != nullptr)
      return a.causal ? launch<IsBf16, 256, true, kModeSparse>(a, s) : launch<IsBf16, 256, false, kModeSparse>(a, s);
    if (!a.causal) return launch<IsBf16, 256, false, kModePlain>(a, s);
    if (a.window < a.N) return launch<IsBf16, 256, true, kModeWindow>(a, s);
    return launch<IsBf16, 256, true, kModePlain>(a, s);
  }
  if (a.d == 128) return dispatch_d<IsBf16, 128>(a, s);
  return a.d == 96 ? dispatch_d<IsBf16, 96>(a, s) : dispatch_d<IsBf16, 64>(a, s);
}

}  // namespace

size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) { return (size_t)(B * H * N) * 8; }
size_t bwd_sparse_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  return SparseWs(B * H, N, d, d).bytes;
}
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) { return dispatch<true>(a, s); }
hipError_t launch_bwd_f16(const BwdArgs& a, hipStream_t s) { return dispatch<false>(a, s); }

}  // namespace fa
