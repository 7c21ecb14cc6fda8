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
#include "mfma_common.hpp"

namespace fa {
namespace {

using namespace mfma;

constexpr int kWaves = 8;          // two waves per SIMD, one workgroup per CU
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kStages = 4;        // LDS ring depth of the K and of the V tiles
constexpr int kBN = 64;           // keys per tile
constexpr int kThreads = 64 * kWaves;

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
  static constexpr int kBytes = kStages * (kKStage + kVStage);
  static_assert(kKStage % 1024 == 0 && kVStage % 1024 == 0, "stages are whole 1 KB loads");
};

// Per-workgroup state and steps of the forward pass.  Everything here is
// device-only; the kernel below only constructs it and runs the tile loop.
//
// Work unit of a wave: 32 query rows against 32-key sub-tiles (two per 64-key
// LDS tile).  One sub-step u issues the score MFMAs of sub-tile u+1 together
// with the exponentials of sub-tile u, then the PV MFMAs of sub-tile u
// together with the mask and maximum of sub-tile u+1.
template <bool IsBf16, int D, bool Causal>
struct FwdBlock {
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using L = Lds<D>;
  static constexpr int kKs = D / 16;  // MFMA k-steps of one 32x32 score block
  static constexpr int kDB = D / 32;  // 32-row blocks of O^T
  static constexpr int kRowBytes = L::kRowBytes;
  static constexpr int kKLoads = L::kKStage / 1024;  // wave-wide 1 KB LDS loads per K tile
  static constexpr int kVLoads = L::kVStage / 1024;
  // K and V loads of one iteration are dealt round-robin to the waves
  static constexpr int kSlots = (kKLoads + kVLoads + kWaves - 1) / kWaves;
  static constexpr uint32_t kNoData = 0x80000000u;  // past any buffer end: reads as zero

  uint8_t* smem;  // K stages 0..kStages-1, then V stages
  const uint8_t* k_ptr;  // K and V of this head (wave-uniform)
  const uint8_t* v_ptr;
  uint32_t head_bytes;
  int N, wave, lane, l32, g, q0, my_q, n_tiles, n_sub;
  float c, tau;
  uint32_t src[kSlots];  // per-lane source byte offset of each load slot
  int k_base, v_base;

  vec8 qf[kKs];       // Q^T B operands: query my_q, d = 16 ks + 8 g + 0..7
  f32x16 acc[kDB];    // O^T: d = 32 db + 8 (r/4) + 4 g + r%4 of query my_q
  float m_ref;        // reference maximum the probabilities are taken against
  float l_part;       // this lane half's share of the denominator
  float mx_next;      // max over this lane half of the next sub-tile's scores

  __device__ __forceinline__ uint8_t* k_stage(int s) const { return smem + s * L::kKStage; }
  __device__ __forceinline__ uint8_t* v_stage(int s) const {
    return smem + kStages * L::kKStage + s * L::kVStage;
  }
  // load slot i of this wave carries combined chunk w + kWaves*i: K chunks
  // first, then V chunks
  __device__ __forceinline__ int slot_chunk(int i) const { return wave + kWaves * i; }

  __device__ __forceinline__ void init(uint8_t* lds, const uint16_t* Q, const uint16_t* K,
                                       const uint16_t* V, int N_, int bh, int qb, float c_,
                                       float tau_, uint32_t q_sign) {
    smem = lds;
    N = N_;
    c = c_;
    tau = tau_;
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
    l32 = lane & 31;
    g = lane >> 5;
    const int64_t head_off = (int64_t)bh * N * D;
    head_bytes = (uint32_t)N * kRowBytes;
    k_ptr = reinterpret_cast<const uint8_t*>(K + head_off);
    v_ptr = reinterpret_cast<const uint8_t*>(V + head_off);

    const int q0_blk = qb * kBM;
    q0 = q0_blk + 32 * wave;
    my_q = q0 + l32;
    const int last_blk_row = min(N, q0_blk + kBM) - 1;
    n_tiles = Causal ? (last_blk_row / kBN + 1) : (N + kBN - 1) / kBN;
    // 32-key sub-tiles this wave computes: all of them, or (causal) those
    // whose first key is not beyond the wave's last row
    const int wave_last_row = min(N, q0 + 32) - 1;
    const int all_sub = (N + 31) / 32;
    n_sub = q0 >= N ? 0 : (Causal ? min(all_sub, wave_last_row / 32 + 1) : all_sub);

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

    // HBM -> LDS copies.  A K tile is kKLoads and a V tile kVLoads wave-wide
    // loads of 1 KB: load c fills LDS bytes [c KB, c KB + 1 KB) of its stage,
    // lane l writing 16 bytes at offset 16 l.  The per-lane source offset picks
    // the (key, 16-byte chunk) that belongs in that slot; slots in row padding
    // get an offset past the buffer end, which reads as zeros.
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int ci = slot_chunk(i);
      if (ci < kKLoads) {
        const int byte = ci * 1024 + lane * 16;
        const int row = byte / L::kKStride, col = byte % L::kKStride;
        src[i] = col < kRowBytes ? (uint32_t)(k_row_key(row) * kRowBytes + col) : kNoData;
      } else {
        const int byte = (ci - kKLoads) * 1024 + lane * 16;
        const int row = byte / L::kVStride, col = byte % L::kVStride;
        src[i] = col < kRowBytes ? (uint32_t)(row * kRowBytes + col) : kNoData;
      }
    }
    // K operand reads (A of S^T): LDS row 32 h + l32 of the tile, 16-byte chunk 2 kk + g.
    k_base = l32 * L::kKStride + g * 16;
    // V operand reads (A of O^T, transpose reads): for 16-key step t of the
    // tile, d-block db and half hh, lane s of each 16-lane group points at key
    // 16 t + 8 g + 4 hh + s/4, columns 32 db + 16 (group & 1) + 4 (s & 3) .. +3;
    // the transpose hands each lane the four keys of its own d column.
    const int grp = lane >> 4, s16 = lane & 15;
    v_base = (8 * g + (s16 >> 2)) * L::kVStride + 2 * (16 * (grp & 1) + 4 * (s16 & 3));

#pragma unroll
    for (int i = 0; i < kDB; ++i) acc[i] = f32x16{};
    m_ref = -INFINITY;
    l_part = 0.f;
    mx_next = -INFINITY;
  }

  // Issue this wave's share of the copies of K tile jk into K stage sk and of
  // V tile jv into V stage sv (tiles past the end are skipped); returns the
  // number of loads issued.
  __device__ __forceinline__ int load_tiles(int jk, int sk, int jv, int sv) const {
    const bool do_k = jk < n_tiles, do_v = jv < n_tiles;
    // resources based at the tile's first row, bounded by the rows left in the
    // head: per-lane offsets are tile-relative and padding slots (offset
    // kNoData >= 2^31) fall outside any bound
    constexpr uint32_t kTileBytes = kBN * kRowBytes;
    const i32x4 tk = make_rsrc(k_ptr + (size_t)jk * kTileBytes, head_bytes - jk * kTileBytes);
    const i32x4 tv = make_rsrc(v_ptr + (size_t)jv * kTileBytes, head_bytes - jv * kTileBytes);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;
    int issued = 0;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int ci = slot_chunk(i);
      if (ci < kKLoads) {
        if (do_k) {
          dma16(tk, lds0 + (uint32_t)(sk * L::kKStage + ci * 1024), src[i]);
          ++issued;
        }
      } else if (ci < kKLoads + kVLoads) {
        if (do_v) {
          dma16(tv, lds0 + (uint32_t)(kStages * L::kKStage + sv * L::kVStage + (ci - kKLoads) * 1024),
                src[i]);
          ++issued;
        }
      }
    }
    return issued;
  }
  // Wait until at most n of this wave's HBM -> LDS loads are outstanding.
  static __device__ __forceinline__ void wait_vm(int n) {
    static_assert(kSlots <= 8, "vmcnt immediates below cover up to 8 loads");
    switch (n) {  // s_waitcnt immediates: vmcnt = n, expcnt and lgkmcnt unchecked
      case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
      case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
      case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
      case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
      case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
      case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
      default: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    }
  }

  __device__ __forceinline__ bool sub_masked(int u) const {
    return (Causal && 32 * u + 31 > q0) || (32 * u + 32 > N);
  }

  // Score block of sub-tile 0 (prologue), masked, and its max.
  __device__ __forceinline__ void first_scores(f32x16& st) {
    const uint8_t* kt = k_stage(0) + k_base;
    st = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk)
      st = E::mfma(*reinterpret_cast<const vec8*>(kt + kk * 32), qf[kk], st);
    mx_next = sub_masked(0) ? mask_max<true>(0, st) : mask_max<false>(0, st);
  }

  // Hide keys of sub-tile u that this lane's query may not see (causal
  // diagonal, sequence end); return the max over this lane half's 16 scores.
  template <bool kMasked>
  __device__ __forceinline__ float mask_max(int u, f32x16& st) const {
    // register r of lane half g holds key 32 u + 16 (r >> 3) + 8 g + (r & 7)
    const int lim = (Causal ? min(my_q, N - 1) : N - 1) - 32 * u - 8 * g;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (kMasked) st[r] = (16 * (r >> 3) + (r & 7)) > lim ? -INFINITY : st[r];
      mx = fmaxf(mx, st[r]);
    }
    return mx;
  }

  // Move the reference maximum only when some row grew by more than tau; the
  // branch is wave-uniform and rarely taken after the first sub-tile.
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

  // Sub-step u, written in issue order.  Phase 1: the score MFMAs of sub-tile
  // u+1 (K operand reads running up to four MFMAs ahead) interleaved with the
  // exponentials of sub-tile u.  Phase 2: the PV MFMAs of sub-tile u (V
  // transpose reads two MFMAs ahead) interleaved with the mask and max of
  // sub-tile u+1.  Scheduling fences keep the VALU work in the shadow of the
  // MFMAs.  k_st / v_st: LDS stages of the K tile holding sub-tile u+1 and of
  // the V tile holding sub-tile u.  On a wave's last sub-tile the scores of
  // "sub-tile u+1" are still formed from whatever that K stage holds and then
  // ignored, so that every sub-step runs the same branch-free phase 1.
  __device__ __forceinline__ void phase1(int u, int k_st, const f32x16& cur, f32x16& nxt,
                                         u32x4 (&pw)[2]) {
    static_assert(kKs == 8 || kKs == 4, "head dim 128 or 64");
    constexpr int kPerMfma = 16 / kKs;  // scores exponentiated per score MFMA
    constexpr int kRing = 4;
    const uint8_t* kt = k_stage(k_st) + k_base + ((u + 1) & 1) * 32 * L::kKStride;
    const float neg_mc = (m_ref == -INFINITY) ? 0.f : -m_ref * c;
    vec8 ka[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ka[i] = *reinterpret_cast<const vec8*>(kt + i * 32);
    float ps[2] = {0.f, 0.f};
    float p_even = 0.f;
#pragma unroll
    for (int i = 0; i < kKs; ++i) {
      nxt = E::mfma(ka[i % kRing], qf[i], i == 0 ? f32x16{} : nxt);
      if (i + kRing < kKs) ka[i % kRing] = *reinterpret_cast<const vec8*>(kt + (i + kRing) * 32);
#pragma unroll
      for (int w = 0; w < kPerMfma; ++w) {
        const int e = i * kPerMfma + w;  // score register 0..15
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[e], c, neg_mc));
        ps[e & 1] += p;
        if (e & 1)
          pw[e >> 3][(e & 7) >> 1] = E::pack2(p_even, p);
        else
          p_even = p;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_part += ps[0] + ps[1];
  }

  template <bool kMaskNext>
  __device__ __forceinline__ void phase2(int u, int v_st, f32x16& nxt, const u32x4 (&pw)[2]) {
    constexpr int kMfmaPV = 2 * kDB;
    const uint8_t* vt = v_stage(v_st) + v_base + (u & 1) * 32 * L::kVStride;
    auto v_frag = [&](int i) {
      const int db = i >> 1, tt = i & 1;
      const uint8_t* vp = vt + 16 * tt * L::kVStride + 64 * db;
      const auto lo = E::read_tr((const lds_void*)vp);
      const auto hi = E::read_tr((const lds_void*)(vp + 4 * L::kVStride));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // register r of lane half g holds key 32 (u+1) + 16 (r >> 3) + 8 g + (r & 7)
    const int lim = (Causal ? min(my_q, N - 1) : N - 1) - 32 * (u + 1) - 8 * g;
    constexpr int kMaxPerMfma = 16 / kMfmaPV;
    vec8 va[2];
    va[0] = v_frag(0);
    va[1] = v_frag(1);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMfmaPV; ++i) {
      acc[i >> 1] = E::mfma(va[i & 1], __builtin_bit_cast(vec8, pw[i & 1]), acc[i >> 1]);
      if (i + 2 < kMfmaPV) va[i & 1] = v_frag(i + 2);
#pragma unroll
      for (int w = 0; w < kMaxPerMfma; ++w) {
        const int r = i * kMaxPerMfma + w;
        if (kMaskNext) nxt[r] = (16 * (r >> 3) + (r & 7)) > lim ? -INFINITY : nxt[r];
        mx = fmaxf(mx, nxt[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mx_next = mx;
  }

  // One sub-step u, if this wave has work for it.  Only each wave's last
  // sub-tile (the causal diagonal, or the ragged end of the sequence) needs a
  // mask; iterations that cannot reach one use the mask-free variant.
  template <bool kMaskable>
  __device__ __forceinline__ void sub(int u, int k_st, int v_st, const f32x16& cur, f32x16& nxt) {
    if (u >= n_sub) return;
    maybe_rescale(mx_next);
    u32x4 pw[2];  // P^T operands (keys 16 tt + 8 g + 0..7 of sub-tile u) as packed pairs
    phase1(u, k_st, cur, nxt, pw);
    if (kMaskable && sub_masked(u + 1))
      phase2<true>(u, v_st, nxt, pw);
    else
      phase2<false>(u, v_st, nxt, pw);
  }

  template <bool kMaskable>
  __device__ __forceinline__ void iteration(int j, f32x16& sa, f32x16& sb) {
    const int s0 = j & 3, s1 = (j + 1) & 3, s2 = (j + 2) & 3, s3 = (j + 3) & 3;
    const int issued = load_tiles(j + 3, s3, j + 2, s2);
    sub<kMaskable>(2 * j, s0, s0, sa, sb);      // next sub-tile: second half of K tile j
    sub<kMaskable>(2 * j + 1, s1, s0, sb, sa);  // next sub-tile: first half of K tile j+1
    wait_vm(issued);
    __syncthreads();
  }

  // Tile loop.  LDS holds rings of kStages K tiles and kStages V tiles.
  // Iteration j consumes sub-tiles 2j and 2j+1: it reads K tiles j (second
  // half) and j+1 (first half) and V tile j.  It issues K tile j+3 (into the
  // stage K tile j-1 left) and V tile j+2 (into the stage V tile j-2 left) and,
  // before its closing barrier, waits only for the loads issued one iteration
  // earlier, so every copy has two iterations to land.
  __device__ __forceinline__ void run(int q0_blk) {
    static_assert(kStages == 4, "the ring arithmetic below assumes four stages");
    f32x16 sa, sb;
    // prologue: K0, V0, K1 resident; K2, V1 in flight; scores of sub-tile 0
    load_tiles(0, 0, 0, 0);
    load_tiles(1, 1, n_tiles, 0);
    const int n1 = load_tiles(2, 2, 1, 1);
    wait_vm(n1);
    __syncthreads();
    if (n_sub > 0) first_scores(sa);

    // first iteration in which some wave's next sub-tile may need a mask
    const int all_sub = (N + 31) / 32;
    const int j_mask = Causal ? max(0, (q0_blk / 32 - 1) / 2)
                              : ((N % 32) ? max(0, (all_sub - 2) / 2) : n_tiles);
    int j = 0;
    for (; j < min(j_mask, n_tiles); ++j) iteration<false>(j, sa, sb);
    for (; j < n_tiles; ++j) iteration<true>(j, sa, sb);
  }

  // O = a / l once; LSE = ln(sum) of the scaled scores
  __device__ __forceinline__ void store(uint16_t* O, float* LSE, int bh) {
    if (n_sub == 0) return;
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
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(
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
  blk.run(qb * kBM);
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
