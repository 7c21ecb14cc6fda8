// Exact attention forward for bf16 / fp16 on gfx950 (MI355X), using MFMA.
//
// What is computed: for every query row, O = softmax(scale * q K^T) V over the
// visible keys and LSE = ln sum exp(scale * q . k), with the N x N scores never
// leaving the chip.  Query blocks are the outer loop and stay resident in
// registers; key/value tiles are the inner loop and stream through LDS
// ("Flash Attention: IO-Aware Exact Attention", section "Loop order changes
// which data is reloaded").  Each query row carries a running maximum, a
// denominator l and an unnormalised d-wide numerator a; when a tile raises the
// maximum, l and a are rescaled by alpha = exp(m_old - m_new), and O = a / l is
// formed once at the end (same page, section "Online softmax makes tiling
// exact", with its remark on FlashAttention-2's unnormalised accumulator).
//
// Mapping to CDNA4:
//  * One workgroup = 4 waves = 128 query rows (32 rows per wave); two
//    workgroups share a CU.  The grid is (query block, batch*head) work items,
//    heaviest causal blocks first so the tail of the launch is short ones.
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 MFMA: the
//    K tile is the A operand (read from LDS), Q^T the B operand (held in
//    registers for the whole loop).  The accumulator then holds one query per
//    lane column, so the row statistics live in that lane: lanes l and l+32
//    share a query and split its keys; the row maximum needs one cross-half
//    permlane exchange, the row sum none until the end.
//  * K rows are placed in LDS in a permuted order chosen so that in the S^T
//    accumulator lane half g holds 8 consecutive keys per 8 registers.  The
//    probabilities, rounded to the input type, are then directly the B operand
//    of O^T += V^T P^T with no LDS round trip.  V stays row-major in LDS and its
//    A operand is gathered with the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16).  O^T keeps the query in the lane column too, so the
//    rescale factor and 1/l are per-lane scalars.
//  * K and V tiles are copied HBM -> LDS by buffer loads that write LDS
//    directly (no register staging); the buffer bounds zero-fill keys past the
//    end of the sequence.  LDS rows are XOR-swizzled in 16-byte chunks so every
//    MFMA operand read is bank-conflict free.
//  * Software pipeline: K runs one tile ahead of V.  While the softmax of
//    tile j runs on the VALU, the score MFMAs of tile j+1 are already issued;
//    tile j+2's K and tile j+1's V are in flight from HBM.
//  * exp is exp2 with scale*log2(e) folded into one FMA per score.  The
//    reference maximum is only moved when a row's maximum grows by more than
//    2^8 in probability units, so most tiles skip the rescale entirely; the
//    result is unchanged (any reference value gives the same a / l and LSE,
//    and probabilities stay below 256).
//  * Causal: tiles entirely above a wave's rows are skipped, the mask is only
//    evaluated on tiles that cross the diagonal or the sequence end.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "fa_internal.hpp"

namespace fa {
namespace {

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

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kThreads = 64 * kWaves;
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

template <bool V> struct BoolTag { static constexpr bool value = V; };

template <bool IsBf16> struct Elt;
template <> struct Elt<true> {
  using scalar = __bf16;
  using vec8 = bf16x8;
  using vec4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 read_tr(const lds_void* p) {
    return __builtin_bit_cast(vec4, read_tr16(p));
  }
};
template <> struct Elt<false> {
  using scalar = _Float16;
  using vec8 = f16x8;
  using vec4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

// LDS row strides (bytes).  K rows carry 16 bytes of padding: the sixteen
// lanes of a 16-byte operand read touch sixteen consecutive rows, which then
// start in sixteen different 4-bank groups.  V rows are read with the transpose
// read, where each 32-lane half touches four consecutive rows over 32
// contiguous bytes per 16-lane group; a 64-byte pad puts those four rows in
// four disjoint 16-bank ranges.
template <int D> struct Lds {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kKStride = kRowBytes + 16;
  static constexpr int kVStride = kRowBytes + 64;
  static constexpr int kKStage = kBN * kKStride;  // multiple of 1 KB
  static constexpr int kVStage = kBN * kVStride;  // multiple of 1 KB
  static constexpr int kBytes = 2 * kKStage + 2 * kVStage;
  static_assert(kKStage % 1024 == 0 && kVStage % 1024 == 0, "stages are whole 1 KB loads");
};

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

// Per-workgroup state and steps of the forward pass.  Everything here is
// device-only; the kernel below only constructs it and runs the tile loop.
template <bool IsBf16, int D, bool Causal>
struct FwdBlock {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using L = Lds<D>;
  static constexpr int kKs = D / 16;  // MFMA k-steps for S^T = K Q^T
  static constexpr int kDB = D / 32;  // 32-row blocks of O^T
  static constexpr int kRowBytes = L::kRowBytes;
  static constexpr int kKLoads = L::kKStage / 1024;  // wave-wide 1 KB LDS loads per K tile
  static constexpr int kVLoads = L::kVStage / 1024;
  static constexpr int kKPerWave = (kKLoads + kWaves - 1) / kWaves;
  static constexpr int kVPerWave = (kVLoads + kWaves - 1) / kWaves;
  static constexpr uint32_t kNoData = 0x80000000u;  // past any buffer end: reads as zero

  uint8_t* smem;  // K stages 0,1 then V stages 0,1
  const uint16_t* Kh;
  const uint16_t* Vh;
  uint32_t head_bytes;
  int N, wave, lane, l32, g, q0, my_q, n_tiles, n_w;
  float c, tau;
  uint32_t k_src[kKPerWave], v_src[kVPerWave];
  int k_base, v_base;

  vec8 qf[kKs];       // Q^T B operands: query my_q, d = 16 ks + 8 g + 0..7
  f32x16 acc[kDB];    // O^T: d = 32 db + 8 (r/4) + 4 g + r%4 of query my_q
  float m_ref;        // reference maximum the probabilities are taken against
  float l_part;       // this lane half's share of the denominator
  f32x16 s_cur[2], s_nxt[2];
  float mx_cur;

  __device__ __forceinline__ uint8_t* k_stage(int s) const { return smem + s * L::kKStage; }
  __device__ __forceinline__ uint8_t* v_stage(int s) const {
    return smem + 2 * L::kKStage + s * L::kVStage;
  }

  __device__ __forceinline__ void init(uint8_t* lds, const uint16_t* Q, const uint16_t* K,
                                       const uint16_t* V, int N_, int bh, int qb, float c_,
                                       float tau_, uint32_t q_sign) {
    smem = lds;
    N = N_;
    c = c_;
    tau = tau_;
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = tid >> 6;
    l32 = lane & 31;
    g = lane >> 5;
    const int64_t head_off = (int64_t)bh * N * D;
    head_bytes = (uint32_t)N * kRowBytes;
    Kh = K + head_off;
    Vh = V + head_off;

    const int q0_blk = qb * kBM;
    q0 = q0_blk + 32 * wave;
    my_q = q0 + l32;
    const int last_blk_row = min(N, q0_blk + kBM) - 1;
    n_tiles = Causal ? (last_blk_row / kBN + 1) : (N + kBN - 1) / kBN;
    const int wave_last_row = min(N, q0 + 32) - 1;
    // tiles this wave computes: all, or (causal) those up to its last row
    n_w = q0 >= N ? 0 : (Causal ? min(n_tiles, wave_last_row / kBN + 1) : n_tiles);

    // Q^T fragments; rows past N read as zeros through the buffer bounds
    const __amdgpu_buffer_rsrc_t q_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Q + head_off), 0, (int)head_bytes, kRsrcFlags);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      u32x4 raw = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rs, my_q * kRowBytes + (2 * ks + g) * 16, 0, 0));
      raw ^= q_sign;  // negative scale: flip the sign of q, exactly
      qf[ks] = __builtin_bit_cast(vec8, raw);
    }

    // HBM -> LDS copies: load i of wave w fills LDS bytes [(w + 4 i) KB, +1 KB)
    // of a stage, lane l writing 16 bytes at offset 16 l.  The per-lane source
    // offset picks the (key, 16-byte chunk) that belongs in that slot; slots in
    // row padding get an offset past the buffer end.
#pragma unroll
    for (int i = 0; i < kKPerWave; ++i) {
      const int byte = (wave + kWaves * i) * 1024 + lane * 16;
      const int row = byte / L::kKStride, col = byte % L::kKStride;
      k_src[i] = col < kRowBytes ? (uint32_t)(k_row_key(row) * kRowBytes + col) : kNoData;
    }
#pragma unroll
    for (int i = 0; i < kVPerWave; ++i) {
      const int byte = (wave + kWaves * i) * 1024 + lane * 16;
      const int row = byte / L::kVStride, col = byte % L::kVStride;
      v_src[i] = col < kRowBytes ? (uint32_t)(row * kRowBytes + col) : kNoData;
    }
    // K operand reads (A of S^T): LDS row kb*32 + l32, 16-byte chunk 2*kk + g.
    k_base = l32 * L::kKStride + g * 16;
    // V operand reads (A of O^T, transpose reads): for key step t, d-block db
    // and half h, lane s of each 16-lane group points at key 16t + 8g + 4h + s/4,
    // columns 32 db + 16 (group & 1) + 4 (s & 3) .. +3; the transpose hands each
    // lane the four keys of its own d column.
    const int grp = lane >> 4, s16 = lane & 15;
    v_base = (8 * g + (s16 >> 2)) * L::kVStride + 2 * (16 * (grp & 1) + 4 * (s16 & 3));

#pragma unroll
    for (int i = 0; i < kDB; ++i) acc[i] = f32x16{};
    m_ref = -INFINITY;
    l_part = 0.f;
    mx_cur = -INFINITY;
  }

  __device__ __forceinline__ void load_k(int j, int s) const {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kh, 0, (int)head_bytes, kRsrcFlags);
    const uint32_t base = (uint32_t)j * kBN * kRowBytes;
#pragma unroll
    for (int i = 0; i < kKPerWave; ++i)
      if (wave + kWaves * i < kKLoads)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void*)(k_stage(s) + (wave + kWaves * i) * 1024), 16,
            k_src[i] == kNoData ? kNoData : base + k_src[i], 0, 0, 0);
  }
  __device__ __forceinline__ void load_v(int j, int s) const {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Vh, 0, (int)head_bytes, kRsrcFlags);
    const uint32_t base = (uint32_t)j * kBN * kRowBytes;
#pragma unroll
    for (int i = 0; i < kVPerWave; ++i)
      if (wave + kWaves * i < kVLoads)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void*)(v_stage(s) + (wave + kWaves * i) * 1024), 16,
            v_src[i] == kNoData ? kNoData : base + v_src[i], 0, 0, 0);
  }
  static __device__ __forceinline__ void wait_loads_and_sync() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS copies have landed
    __syncthreads();
  }

  // S^T of the tile in K stage s
  __device__ __forceinline__ void compute_s(int s, f32x16 (&st)[2]) const {
    const uint8_t* kt = k_stage(s) + k_base;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < kKs; ++kk) {
        const vec8 a = *reinterpret_cast<const vec8*>(kt + kb * 32 * L::kKStride + kk * 32);
        st[kb] = E::mfma(a, qf[kk], st[kb]);
      }
    }
  }

  __device__ __forceinline__ bool tile_masked(int j) const {
    return (Causal && j * kBN + kBN - 1 > q0) || (j * kBN + kBN > N);
  }

  // Hide the keys of tile j this lane's query may not see (causal diagonal,
  // sequence end) and return the max over this lane half's 32 scores.
  template <bool kMasked>
  __device__ __forceinline__ float mask_and_max(int j, f32x16 (&st)[2]) const {
    // register r of lane half g holds key j*64 + kb*32 + 16*(r>>3) + 8g + (r&7);
    // it is visible iff that offset is <= lim
    const int lim = (Causal ? min(my_q, N - 1) : N - 1) - j * kBN - 8 * g;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kMasked) {
          const int off = kb * 32 + 16 * (r >> 3) + (r & 7);
          st[kb][r] = off > lim ? -INFINITY : st[kb][r];
        }
        mx = fmaxf(mx, st[kb][r]);
      }
    return mx;
  }

  // Move the reference maximum only when some row grew by more than tau; the
  // branch is wave-uniform and rarely taken after the first tile.
  __device__ __forceinline__ void maybe_rescale(float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + tau) != 0) {
      const float m_row = fmaxf(m_ref, xhalf_max(mx));
      const float m_new = (m_row > m_ref + tau) ? m_row : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
      m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db) acc[db] *= alpha;
    }
  }

  // p = exp2(c s - c m_ref) for the tile's 32 scores per lane (hidden scores
  // are -inf and give 0), summed into l and rounded into the four P^T
  // operands: step t covers keys 16t..16t+15, lane half g holds 8 of them.
  __device__ __forceinline__ void exp_tile(const f32x16 (&st)[2], vec8 (&pb)[4]) {
    const float neg_mc = (m_ref == -INFINITY) ? 0.f : -m_ref * c;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[t >> 1][8 * (t & 1) + e], c, neg_mc));
        pf[e] = p;
        ps[e & 3] += p;
      }
      pb[t] = __builtin_convertvector(pf, vec8);
    }
    l_part += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  }

  // O^T += V^T P^T for tile j
  __device__ __forceinline__ void pv_tile(int j, const vec8 (&pb)[4]) {
    const uint8_t* vt = v_stage(j & 1) + v_base;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint8_t* vp = vt + 16 * t * L::kVStride + 64 * db;
        const auto lo = E::read_tr((const lds_void*)vp);
        const auto hi = E::read_tr((const lds_void*)(vp + 4 * L::kVStride));
        const vec8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = E::mfma(a, pb[t], acc[db]);
      }
  }

  // One step for tile j when tile j+1 also has work: the score MFMAs of tile
  // j+1 are issued together with the exponentials of tile j, then the PV
  // MFMAs of tile j together with the mask and max of tile j+1.
  template <bool kMaskNext>
  __device__ __forceinline__ void pipelined_step(int j) {
    vec8 pb[4];
    compute_s((j + 1) & 1, s_nxt);
    exp_tile(s_cur, pb);
    pv_tile(j, pb);
    mx_cur = mask_and_max<kMaskNext>(j + 1, s_nxt);
    s_cur[0] = s_nxt[0];
    s_cur[1] = s_nxt[1];
  }

  __device__ __forceinline__ void last_step(int j) {
    vec8 pb[4];
    exp_tile(s_cur, pb);
    pv_tile(j, pb);
  }

  __device__ __forceinline__ void run() {
    // prologue: K0, V0, K1 in LDS; S0 computed and masked
    load_k(0, 0);
    load_v(0, 0);
    if (n_tiles > 1) load_k(1, 1);
    wait_loads_and_sync();
    if (n_w > 0) {
      compute_s(0, s_cur);
      mx_cur = tile_masked(0) ? mask_and_max<true>(0, s_cur) : mask_and_max<false>(0, s_cur);
    }
    __syncthreads();  // K stage 0 is refilled in iteration 0

    // K of tile j+2 and V of tile j+1 stream in while tile j is consumed
    for (int j = 0; j < n_tiles; ++j) {
      if (j + 2 < n_tiles) load_k(j + 2, j & 1);
      if (j + 1 < n_tiles) load_v(j + 1, (j + 1) & 1);
      if (j < n_w) {
        maybe_rescale(mx_cur);
        if (j + 1 < n_w) {
          if (tile_masked(j + 1))
            pipelined_step<true>(j);
          else
            pipelined_step<false>(j);
        } else {
          last_step(j);
        }
      }
      wait_loads_and_sync();
    }
  }

  // O = a / l once; LSE = ln(sum) of the scaled scores
  __device__ __forceinline__ void store(uint16_t* O, float* LSE, int bh) {
    if (n_w == 0) return;
    const float l_tot = xhalf_sum(l_part);
    const float inv = 1.0f / l_tot;
    if (my_q >= N) return;
    uint16_t* orow = O + (int64_t)bh * N * D + (int64_t)my_q * D;
    typedef __attribute__((ext_vector_type(4))) typename E::scalar h4_t;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v4 = {acc[db][4 * gq] * inv, acc[db][4 * gq + 1] * inv,
                          acc[db][4 * gq + 2] * inv, acc[db][4 * gq + 3] * inv};
        const auto h4 = __builtin_convertvector(v4, h4_t);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * gq + 4 * g) = __builtin_bit_cast(u32x2, h4);
      }
    if (LSE != nullptr && g == 0)
      LSE[(int64_t)bh * N + my_q] =
          ((m_ref == -INFINITY ? 0.f : m_ref * c) + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
};

template <bool IsBf16, int D, bool Causal>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int BH, int n_qblocks, float c,
    float tau, uint32_t q_sign) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Lds<D>::kBytes];
  // work item: (query block, batch*head); heaviest causal blocks first
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (Causal) qb = n_qblocks - 1 - qb;
  FwdBlock<IsBf16, D, Causal> blk;
  blk.init(smem, Q, K, V, N, bh, qb, c, tau, q_sign);
  blk.run();
  blk.store(O, LSE, bh);
}

template <bool IsBf16, int D, bool Causal>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int N = (int)a.N;
  const int BH = (int)(a.B * a.H);
  const int n_qblocks = (N + kBM - 1) / kBM;
  const dim3 grid((unsigned)(n_qblocks * BH));
  // c = |scale| * log2(e).  A zero scale is run as the limit scale -> 0+:
  // with c = 1e-30 every exp2 argument c*(s - m) rounds to exactly 0 in fp32,
  // so all visible keys weigh exactly 1 and hidden ones (-inf) weigh 0.
  const float c = a.scale != 0.f ? __builtin_fabsf(a.scale) * 1.4426950408889634f : 1e-30f;
  // reference-maximum slack: 8 in log2 units, i.e. probabilities up to 2^8
  const float tau = 8.0f / c;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<IsBf16, D, Causal>), grid, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, N, BH,
                     n_qblocks, c, tau, q_sign);
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
