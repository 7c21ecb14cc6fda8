// Exact attention forward for bf16 / fp16 on gfx950 (MI355X), d = d_v = 64,
// using the 32x32x16 MFMA.
//
// The same computation and the same workgroup, copy and softmax design as the
// main forward kernel (fwd_mfma.hip): for every query row, O = softmax(scale *
// q K^T) V over the visible keys and LSE = ln sum exp(scale * q . k), with the
// N x N scores never leaving the chip ("Flash Attention: IO-Aware Exact
// Attention", sections "Loop order changes which data is reloaded" and
// "Online softmax makes tiling exact").  It differs in the MFMA shape.  At
// d = 64 a 32-key block holds only 8 products of the 32x32x16 shape beside the
// same softmax work as at d = 128, so the block is bound by VALU issue rather
// than by the matrix cores; the main kernel's 16x16x32 shape, which lowers the
// chip's power per product, would double the MFMA instructions that compete
// for that issue, and measured about 5 % slower on B=8, H=12, N=1024.
//
// Mapping to CDNA4:
//  * One workgroup = 8 waves = 256 query rows (32 rows per wave), one
//    workgroup per CU, two waves per SIMD.  The grid is (query block,
//    batch*head) work items, heaviest causal blocks first so the tail of the
//    launch is short ones.
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 MFMA: the
//    K tile is the A operand (read from LDS), Q^T the B operand (held in
//    registers for the whole loop).  The accumulator then holds one query per
//    lane column, so the row statistics live in that lane: lanes l and l+32
//    share a query and split its keys.
//  * K rows are placed in LDS in a permuted order chosen so that in the S^T
//    accumulator lane half g holds 8 consecutive keys per 8 registers.  The
//    probabilities, rounded to the input type, are then directly the B operand
//    of O^T += V^T P^T with no LDS round trip.  V stays row-major in LDS and its
//    A operand is gathered with the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16).  O^T keeps the query in the lane column too, so the
//    rescale factor and 1/l are per-lane scalars.
//  * K and V tiles are copied HBM -> LDS by buffer loads that write LDS
//    directly (no register staging); the buffer bounds zero-fill keys past the
//    end of the sequence.  Every wave issues the same number of copies per
//    tile step, so the copy code has no branches.
//  * Work of a wave is a chain of 32-key blocks.  Block u issues the PV MFMAs
//    of sub-tile u-1 and the score MFMAs of sub-tile u+1, and spreads the
//    exponentials of sub-tile u between them, so no MFMA of a block waits for
//    that block's VALU work.  The K operand of sub-tile u+1 is read from LDS at
//    the start of block u, the V operand of sub-tile u during its second half.
//  * exp is exp2 with scale*log2(e) folded into one FMA per score.  The
//    probabilities of a block are taken against the current reference maximum
//    without first computing the block's own maximum; the block's fp32
//    partial row sums reveal whether any probability may exceed the cap
//    (2^15 for fp16, 2^24 for bf16, kSumCap below), and only then is the
//    reference raised to the true running maximum, a and l rescaled and the
//    block's probabilities recomputed.  Any reference value gives the same
//    a / l and LSE; the check keeps every probability below the cap.
//  * Causal: tiles entirely above a wave's rows are skipped, the mask is only
//    evaluated on blocks that cross the diagonal or the sequence end.
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
// A block whose partial row sum (16 probabilities of one lane half) exceeds
// the cap moves the reference maximum, so every probability stays below it:
// 2^15 for fp16, whose P operand reaches 65504, and 2^24 for bf16, which has
// the fp32 exponent range.  The probabilities' relative precision does not
// depend on their size, so a high cap only makes the costly raise rarer (with
// sharp rows, scores of std 9, a cap of 2^8 raised the reference often enough
// to slow the forward by about a fifth).  The price is range: the fp32
// numerator sum of up to N probabilities times |V| must stay finite, which for
// bf16 values bounds |V| by about 2^104 / N.
template <bool IsBf16> constexpr float kSumCap = IsBf16 ? 16777216.0f : 32768.0f;
// Exponent offset of a row that has no reference yet (every key seen so far
// hidden): any visible score then gives probability +inf, so the row sum
// exceeds kSumCap and the block moves the reference; a hidden one gives 0.
constexpr float kNoRef = 1e30f;
// Masks a block of scores may need: none, the causal diagonal and the
// sequence end, or those and the left edge of a sliding window.
constexpr int kMaskNone = 0, kMaskEdge = 1, kMaskWindow = 2;
// Block-sparse: a workgroup's list of key tiles (index | query-block bits <<
// 16, see compact_tiles) lives in LDS after the rings.

// LDS row strides (bytes).  K rows carry 16 bytes of padding: the sixteen
// lanes of a 16-byte operand read touch sixteen consecutive rows, which then
// start in sixteen different 4-bank groups.  V rows are read with the transpose
// read, where each 32-lane half touches four consecutive rows over 32
// contiguous bytes per 16-lane group; a 64-byte pad puts those four rows in
// four disjoint 16-bank ranges.  One extra 1 KB slot at the end absorbs the
// copies of waves that have no real chunk for their last copy slot.  Only
// d = d_v = 64 is launched from this source.
template <int D, int DV = D> struct Lds {
  static constexpr int kRowBytes = 2 * D;    // a K (and Q) row
  static constexpr int kVRowBytes = 2 * DV;  // a V (and O) row
  static constexpr int kKStride = (D == 96 ? 256 : kRowBytes) + 16;
  static constexpr int kVStride = (DV == 96 ? 256 : kVRowBytes) + 64;
  static constexpr int kKStage = kBN * kKStride;  // multiple of 1 KB
  static constexpr int kVStage = kBN * kVStride;  // multiple of 1 KB
  static constexpr int kSink = kStages * (kKStage + kVStage);
  static constexpr int kBytes = kSink + 1024;
  static_assert(kKStage % 1024 == 0 && kVStage % 1024 == 0, "stages are whole 1 KB loads");
  static_assert(kBytes <= 160 * 1024, "fits the 160 KB LDS of a CU");
};

// Per-workgroup state and steps of the forward pass.  Everything here is
// device-only; the kernel below only constructs it and runs the tile loop.
// Mode kModeWindow (causal only) adds a sliding window narrower than the
// sequence: key j is visible to query i iff i - win < j <= i.  Mode
// kModeSparse adds a block-sparse mask: key j is visible to query i iff the
// mask byte of (query block i / 64, key block j / 64) is nonzero.
template <bool IsBf16, int D, bool Causal, int Mode, int DV = D>
struct FwdBlock {
  static constexpr bool kWin = Causal && Mode == kModeWindow;
  static constexpr bool kSparse = Mode == kModeSparse;
  static_assert(kBN == kSparseBlock && kBM % kSparseBlock == 0, "mask blocks are key tiles");
  using E = Elt<IsBf16>;
  using vec8 = typename E::vec8;
  using L = Lds<D, DV>;
  static constexpr int kKs = D / 16;   // score MFMAs of one 32x32 block (k-steps over d)
  static constexpr int kDB = DV / 32;  // 32-row blocks of O^T
  static constexpr int kPV = 2 * kDB;  // PV MFMAs of one 32-key block
  static constexpr int kRowBytes = L::kRowBytes;
  // HBM -> LDS copies: a K tile is kKLoads and a V tile kVLoads wave-wide
  // 1 KB copies.  Wave w copies K chunks w + 8 i and V chunks w + 8 i of the
  // whole-round parts, plus one extra chunk: the V remainder goes to waves
  // 0.., the K remainder to the waves after them, and the rest copy zeros into
  // the sink slot.
  static constexpr int kKLoads = L::kKStage / 1024;
  static constexpr int kVLoads = L::kVStage / 1024;
  static constexpr int kFullK = kKLoads / kWaves, kFullV = kVLoads / kWaves;
  static constexpr int kRemK = kKLoads % kWaves, kRemV = kVLoads % kWaves;
  static_assert(kRemK + kRemV <= kWaves, "one extra copy per wave covers the remainders");
  static constexpr int kCopies = kFullK + kFullV + 1;  // copies per wave per tile step
  static_assert(kFullK >= 1 && kFullK <= 2 && kFullV >= 1 && kFullV <= 2, "copy groups of 3 to 5");
  static constexpr uint32_t kNoData = 0x80000000u;    // past any buffer end: reads as zero

  uint8_t* smem;  // K stages 0..kStages-1, then V stages, then the sink slot
  const uint8_t* k_ptr;  // K and V of this head (wave-uniform)
  const uint8_t* v_ptr;
  uint32_t head_bytes;   // extent of one head's rows in k: (N - 1) rows + one row of data
  uint32_t row_bytes;    // distance of consecutive rows of k
  uint32_t v_head_bytes, v_row_bytes;  // the same for v
  int64_t o_off;         // this head's first output element, and the output row stride
  int64_t o_sn;
  int N, win, wave, lane, l32, g, q0, my_q, n_tiles, n_sub;
  int u_lo;   // first 32-key block this wave computes (sliding window)
  // block-sparse: the workgroup's key tiles in LDS, their count, and the bit
  // of this wave's 64-row query block in a list entry
  const uint32_t* tiles;
  int n_pos, qbit;
  bool live;  // block-sparse: the wave computed the previous list position
  float c;
  uint32_t src_k[kFullK], src_v[kFullV], src_x;  // per-lane source offsets of the copies
  // The extra copy writes LDS byte x_off + (K stage offset & x_kmask) +
  // (V stage offset & x_vmask), reading the V tile iff x_vmask != 0 (a copy
  // into the sink reads nothing: its source offset is past every buffer).
  uint32_t x_off, x_kmask, x_vmask;
  int k_base, v_base;

  vec8 qf[kKs];       // Q^T B operands: query my_q, d = 16 ks + 8 g + 0..7
  f32x16 acc[kDB];    // O^T: d = 32 db + 8 (r/4) + 4 g + r%4 of query my_q
  float m_ref;        // reference maximum the probabilities are taken against
  float neg_mc;       // -m_ref * c, or kNoRef while m_ref = -inf
  float l_part;       // this lane half's share of the denominator
  f32x16 s_cur;       // scores of the block being exponentiated
  u32x4 p_prev[2];    // probabilities of the previous block (B operands)
  vec8 vfr[kPV];      // V^T operands of the previous block

  __device__ __forceinline__ const uint8_t* k_stage(int s) const { return smem + s * L::kKStage; }
  __device__ __forceinline__ const uint8_t* v_stage(int s) const {
    return smem + kStages * L::kKStage + s * L::kVStage;
  }

  // per-lane source offset of copy chunk ci of a K (is_v = false) or V tile
  __device__ __forceinline__ uint32_t chunk_src(bool is_v, int ci) const {
    const int stride = is_v ? L::kVStride : L::kKStride;
    const int byte = ci * 1024 + lane * 16;
    const int row = byte / stride, col = byte % stride;
    if (col >= (is_v ? L::kVRowBytes : kRowBytes)) return kNoData;  // row padding
    return is_v ? (uint32_t)row * v_row_bytes + (uint32_t)col
                : (uint32_t)k_row_key(row) * row_bytes + (uint32_t)col;
  }

  __device__ __forceinline__ void init(uint8_t* lds, const uint16_t* Q, const uint16_t* K,
                                       const uint16_t* V, int N_, int win_, int H, int bh, int qb,
                                       float c_, uint32_t q_sign, const Layout& lq, const Layout& in,
                                       const Layout& lv, const Layout& out) {
    smem = lds;
    N = N_;
    win = win_;
    c = c_;
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
    l32 = lane & 31;
    g = lane >> 5;
    const int b = bh / H, h = bh - b * H;
    const int64_t head_off = b * in.sb + h * in.sh;
    row_bytes = (uint32_t)(2 * in.sn);
    head_bytes = (uint32_t)(N - 1) * row_bytes + (uint32_t)kRowBytes;
    v_row_bytes = (uint32_t)(2 * lv.sn);
    v_head_bytes = (uint32_t)(N - 1) * v_row_bytes + (uint32_t)L::kVRowBytes;
    o_off = b * out.sb + h * out.sh;
    o_sn = out.sn;
    k_ptr = reinterpret_cast<const uint8_t*>(K + head_off);
    v_ptr = reinterpret_cast<const uint8_t*>(V + (b * lv.sb + h * lv.sh));

    const int q0_blk = qb * kBM;
    q0 = q0_blk + 32 * wave;
    my_q = q0 + l32;
    const int last_blk_row = min(N, q0_blk + kBM) - 1;
    n_tiles = Causal ? (last_blk_row / kBN + 1) : (N + kBN - 1) / kBN;
    // 32-key blocks this wave computes: all of them, or (causal) those whose
    // first key is not beyond the wave's last row
    const int wave_last_row = min(N, q0 + 32) - 1;
    const int all_sub = (N + 31) / 32;
    n_sub = q0 >= N ? 0 : (Causal ? min(all_sub, wave_last_row / 32 + 1) : all_sub);
    // blocks before the window of the wave's first query are skipped
    u_lo = kWin ? max(0, q0 - win + 1) / 32 : 0;

    // Q^T fragments; rows past N read as zeros through the buffer bounds
    const uint32_t q_row_bytes = (uint32_t)(2 * lq.sn);
    const __amdgpu_buffer_rsrc_t q_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Q + (b * lq.sb + h * lq.sh)), 0, (int)((uint32_t)(N - 1) * q_row_bytes + kRowBytes),
        kRsrcFlags);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      u32x4 raw = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rs, (int)((uint32_t)my_q * q_row_bytes) + (2 * ks + g) * 16, 0, 0));
      raw ^= q_sign;  // negative scale: flip the sign of q, exactly
      qf[ks] = __builtin_bit_cast(vec8, raw);
    }

#pragma unroll
    for (int i = 0; i < kFullK; ++i) src_k[i] = chunk_src(false, wave + kWaves * i);
#pragma unroll
    for (int i = 0; i < kFullV; ++i) src_v[i] = chunk_src(true, wave + kWaves * i);
    if (wave < kRemV) {  // a chunk of the V remainder
      const int ci = kFullV * kWaves + wave;
      x_off = ci * 1024;
      x_kmask = 0u;
      x_vmask = ~0u;
      src_x = chunk_src(true, ci);
    } else if (wave < kRemV + kRemK) {  // a chunk of the K remainder
      const int ci = kFullK * kWaves + wave - kRemV;
      x_off = ci * 1024;
      x_kmask = ~0u;
      x_vmask = 0u;
      src_x = chunk_src(false, ci);
    } else {  // zeros into the sink
      x_off = L::kSink;
      x_kmask = 0u;
      x_vmask = 0u;
      src_x = kNoData;
    }

    // K operand reads (A of S^T): LDS row 32 h + l32 of the tile, 16-byte chunk 2 kk + g.
    k_base = l32 * L::kKStride + g * 16;
    // V operand reads (A of O^T, transpose reads): for 16-key step t of the
    // block, d-block db and half hh, lane s of each 16-lane group points at key
    // 16 t + 8 g + 4 hh + s/4, columns 32 db + 16 (group & 1) + 4 (s & 3) .. +3;
    // the transpose hands each lane the four keys of its own d column.
    const int grp = lane >> 4, s16 = lane & 15;
    v_base = (8 * g + (s16 >> 2)) * L::kVStride + 2 * (16 * (grp & 1) + 4 * (s16 & 3));

#pragma unroll
    for (int i = 0; i < kDB; ++i) acc[i] = f32x16{};
    m_ref = -INFINITY;
    neg_mc = kNoRef;
    l_part = 0.f;
    if (kWin || kSparse) {
      // A wave whose window starts after the workgroup's first step (or a
      // block-sparse run) begins with a normal block: zeros make its PV MFMAs
      // add 0, and kNoRef sends it down the reference-update path.
      s_cur = f32x16{};
      p_prev[0] = p_prev[1] = u32x4{};
#pragma unroll
      for (int i = 0; i < kPV; ++i) vfr[i] = vec8{};
    }
  }

  // Copies of K tile jk into K stage sk and V tile jv into V stage sv (a tile
  // at or past n_tiles copies zeros: its buffer is empty): buffer ranges and
  // LDS destinations, all wave-uniform.  Every wave issues exactly kCopies
  // copies, either at once (load_tiles) or one by one (copy_one).
  struct Copies {
    i32x4 tk, tv, tx;
    uint32_t k_st, v_st, x_lds;
  };
  __device__ __forceinline__ Copies prepare_tiles(int jk, int sk, int jv, int sv) const {
    const uint32_t tile_bytes = kBN * row_bytes, v_tile_bytes = kBN * v_row_bytes;
    const uint32_t k_left = jk < n_tiles ? head_bytes - (uint32_t)jk * tile_bytes : 0u;
    const uint32_t v_left = jv < n_tiles ? v_head_bytes - (uint32_t)jv * v_tile_bytes : 0u;
    const i32x4 tk = make_rsrc(k_ptr + (size_t)jk * tile_bytes, k_left);
    const i32x4 tv = make_rsrc(v_ptr + (size_t)jv * v_tile_bytes, v_left);
    // wave-uniform by construction; readfirstlane keeps the selection in SGPRs
    i32x4 tx;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      tx[w] = __builtin_amdgcn_readfirstlane((int)(((uint32_t)tk[w] & ~x_vmask) | ((uint32_t)tv[w] & x_vmask)));
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)smem + (uint32_t)(wave * 1024);
    const uint32_t k_st = base + (uint32_t)(sk * L::kKStage);
    const uint32_t v_st = base + (uint32_t)(kStages * L::kKStage + sv * L::kVStage);
    const uint32_t x_lds = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)((uint32_t)(uintptr_t)(lds_void*)smem + x_off + ((uint32_t)(sk * L::kKStage) & x_kmask) +
              ((uint32_t)(kStages * L::kKStage + sv * L::kVStage) & x_vmask)));
    return Copies{tk, tv, tx, k_st, v_st, x_lds};
  }
  // Copy i of a prepared set: K chunks first, then V chunks, then the extra one.
  __device__ __forceinline__ void copy_one(const Copies& cp, int i) const {
    if (i < kFullK)
      dma16(cp.tk, cp.k_st + (uint32_t)(i * kWaves * 1024), src_k[i]);
    else if (i < kFullK + kFullV)
      dma16(cp.tv, cp.v_st + (uint32_t)((i - kFullK) * kWaves * 1024), src_v[i - kFullK]);
    else
      dma16(cp.tx, cp.x_lds, src_x);
  }
  // All copies at once, in one asm statement that saves and restores M0 once.
  __device__ __forceinline__ void load_tiles(int jk, int sk, int jv, int sv) const {
    const Copies cp = prepare_tiles(jk, sk, jv, sv);
    const i32x4 &tk = cp.tk, &tv = cp.tv, &tx = cp.tx;
    const uint32_t k_st = cp.k_st, v_st = cp.v_st, x_lds = cp.x_lds;
    if constexpr (kFullK == 2 && kFullV == 2)
      dma_group5(tk, tv, tx, k_st, k_st + kWaves * 1024, v_st, v_st + kWaves * 1024, x_lds,
                 src_k[0], src_k[1], src_v[0], src_v[1], src_x);
    else if constexpr (kFullK == 2)
      dma_group4a(tk, tv, tx, k_st, k_st + kWaves * 1024, v_st, x_lds, src_k[0], src_k[1],
                  src_v[0], src_x);
    else if constexpr (kFullV == 2)
      dma_group4b(tk, tv, tx, k_st, v_st, v_st + kWaves * 1024, x_lds, src_k[0], src_v[0],
                  src_v[1], src_x);
    else
      dma_group3(tk, tv, tx, k_st, v_st, x_lds, src_k[0], src_v[0], src_x);
  }
  // Wait until at most one tile step's copies of this wave are outstanding.
  static __device__ __forceinline__ void wait_older_copies() {
    static_assert(kCopies >= 1 && kCopies <= 15, "vmcnt immediate");
    // s_waitcnt immediate: vmcnt = kCopies (low 4 bits), expcnt and lgkmcnt unchecked
    __builtin_amdgcn_s_waitcnt(0x0F70 | kCopies);
  }

  // Key tile at list position p (block-sparse), or n_tiles (zeros) past its end.
  __device__ __forceinline__ int tile_at(int p) const {
    return p < n_pos ? __builtin_amdgcn_readfirstlane((int)(tiles[p] & 0xFFFFu)) : n_tiles;
  }
  // First key of 32-key block u (block-sparse: block u is half u & 1 of the
  // tile at list position u / 2).
  __device__ __forceinline__ int kpos(int u) const {
    return kSparse ? kBN * tile_at(u >> 1) + 32 * (u & 1) : 32 * u;
  }

  // Hide keys of block u that this lane's query may not see: the causal
  // diagonal and the sequence end; with kMaskWindow also keys left of the
  // query's sliding window.
  template <int kMask>
  __device__ __forceinline__ void apply_mask(int u, f32x16& st) const {
    // register r of lane half g holds key kpos(u) + 16 (r >> 3) + 8 g + (r & 7)
    const int k0 = kpos(u);
    // Wave-uniform: a block whose keys every row of the wave sees (none past
    // the first row's diagonal or the sequence end, none left of the last
    // row's window) needs no selects.  In a step that may need masks only a
    // wave's diagonal block (and a block at the sequence end or the window
    // edge) does.
    const bool cut_right = k0 + 31 > (Causal ? min(q0, N - 1) : N - 1);
    const bool cut_left = kMask == kMaskWindow && kWin && k0 <= q0 + 31 - win;
    if (!cut_right && !cut_left) return;
    const int lim = (Causal ? min(my_q, N - 1) : N - 1) - k0 - 8 * g;
    const int lo = my_q - win + 1 - k0 - 8 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = 16 * (r >> 3) + (r & 7);
      const bool hide = (kMask == kMaskWindow && kWin) ? (o > lim || o < lo) : o > lim;
      st[r] = hide ? -INFINITY : st[r];
    }
  }

  // Probabilities of scores 2e, 2e+1 against the current reference, packed
  // into the B operand and added (in fp32) to a partial row sum.
  __device__ __forceinline__ void exp_pair(const f32x16& st, int e, u32x4 (&pw)[2], float& sum) const {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * e], c, neg_mc));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * e + 1], c, neg_mc));
    pw[e >> 2][e & 3] = E::pack2(p0, p1);
    sum += p0 + p1;
  }

  // Raise the reference to the running maximum over the scores st (both lane
  // halves), rescale a and l, and leave neg_mc matching.
  __device__ __forceinline__ void raise_reference(const f32x16& st) {
    float mx = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
    const float m_new = fmaxf(m_ref, xhalf_max(mx));
    const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
    m_ref = m_new;
    neg_mc = (m_new == -INFINITY) ? kNoRef : -m_new * c;
    l_part *= alpha;
#pragma unroll
    for (int db = 0; db < kDB; ++db) acc[db] *= alpha;
  }

  // Scores of block u (K tile u/2, half u&1, still resident in LDS during the
  // tile step that holds block u), masked when kMask.
  template <int kMask>
  __device__ __forceinline__ f32x16 scores(int u) const {
    const uint8_t* kt = k_stage((u >> 1) & 3) + k_base + (u & 1) * 32 * L::kKStride;
    f32x16 st = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kKs; ++kk)
      st = E::mfma(*reinterpret_cast<const vec8*>(kt + kk * 32), qf[kk], st);
    if (kMask != kMaskNone) apply_mask<kMask>(u, st);
    return st;
  }

  // MFMA slot of step st (0 scale, 1 exp2, 2 pack and partial sum) of score
  // pair e, for blocks of 8 MFMA slots (or 4, a wave's first block).  Steps
  // that land in the same slot run in program order.
  template <int kSlots>
  static constexpr int slot_of(int e, int st) {
    static_assert(kSlots == 8 || kSlots == 4, "d = 64 blocks hold 8 or 4 MFMAs");
    return kSlots == 8 ? e / 2 + st : (e / 4 + st < 3 ? e / 4 + st : 3);
  }

  // Block u: PV MFMAs of block u-1 (none if kFirst), score MFMAs of block u+1,
  // and between them the probabilities of block u.  On entry s_cur holds the
  // scores of block u, p_prev / vfr the operands of block u-1.  The K operand
  // read for score MFMA i is issued right after PV MFMA i, the V operand read
  // for next block's PV MFMA i right after score MFMA i: every operand is read
  // a full phase before its use, and each read reuses the registers of the
  // operand the preceding MFMA just consumed.  On a wave's last block the
  // scores of "block u+1" are still formed from whatever the K stage holds and
  // never used, so every block runs the same code.
  //
  // A wave's first block is either kFirst (its scores were formed in the
  // prologue and it sets the reference from them), or, for a wave whose
  // sliding window starts after the workgroup's first tile step, a normal
  // block: the zeros in s_cur, seen against kNoRef, send it down the
  // reference-update path, which forms its scores from LDS, while
  // p_prev = vfr = 0 make its PV MFMAs add 0.
  //
  // kHalf (0 or 1) is the block's place in its tile step; it sets the wave's
  // issue priority (see step()).
  template <int kMask, bool kFirst = false, int kHalf = 0, bool kCopy = false>
  __device__ __forceinline__ void block(int u, const Copies* cp = nullptr) {
    constexpr int kMfmas = (kFirst ? 0 : kPV) + kKs;
    static_assert(kMfmas == 8 || kMfmas == 4, "slot schedules exist for 4 and 8 MFMAs");
    auto slot = [](int e, int st) { return slot_of<kMfmas>(e, st); };
    // K operand of block u+1: K tile (u+1)/2, half (u+1)&1
    const uint8_t* kt = k_stage(((u + 1) >> 1) & 3) + k_base + ((u + 1) & 1) * 32 * L::kKStride;
    // V operand of block u (for the next block's PV MFMAs): V tile u/2, half u&1.
    // The stage offset is hidden from the compiler (an empty asm on an SGPR)
    // so that it is not folded into the reads' constant offsets: past 64 KB
    // they no longer fit the 16-bit LDS offset field and every read would
    // need an address add of its own.
    uint32_t v_off = kStages * L::kKStage + ((u >> 1) & 3) * L::kVStage + (u & 1) * 32 * L::kVStride;
    asm("" : "+s"(v_off));
    const uint8_t* vt = smem + v_off + v_base;
    vec8 kfr[kKs];
    if (kFirst) {
#pragma unroll
      for (int i = 0; i < kKs; ++i) kfr[i] = *reinterpret_cast<const vec8*>(kt + i * 32);
    }
    if (kMask != kMaskNone) apply_mask<kMask>(u, s_cur);
    if (kFirst) raise_reference(s_cur);  // the first block sets the reference outright

    u32x4 pw[2];
    float sum[2];  // partial row sums of even and odd score pairs
    f32x16 s_next;
    float pr[16];  // scaled scores, then probabilities
#pragma unroll
    for (int t = 0; t < kMfmas; ++t) {
      if (!kFirst && t < kPV) {
        // PV order 0, 2, 4, .., 1, 3, ..: no two adjacent MFMAs share an
        // accumulator, and the operands of the second key half come last
        const int f = (t < kPV / 2) ? 2 * t : 2 * (t - kPV / 2) + 1;
        acc[f >> 1] = E::mfma(vfr[f], __builtin_bit_cast(vec8, p_prev[f & 1]), acc[f >> 1]);
        // K operands r = t, t + kPV, ..: all are read in the PV phase
#pragma unroll
        for (int r = t; r < kKs; r += kPV) kfr[r] = *reinterpret_cast<const vec8*>(kt + r * 32);
      } else {
        const int i = kFirst ? t : t - kPV;  // score k-step
        s_next = E::mfma(kfr[i], qf[i], i == 0 ? f32x16{} : s_next);
        // V^T operands f = i, i + kKs, .. of block u: two transpose reads each
#pragma unroll
        for (int f = i; f < kPV; f += kKs) {
          const int db = f >> 1, tt = f & 1;
          const uint8_t* vp = vt + 16 * tt * L::kVStride + 64 * db;
          const auto lo = E::read_tr((const lds_void*)vp);
          const auto hi = E::read_tr((const lds_void*)(vp + 4 * L::kVStride));
          vfr[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
      // the tile step's copies, spread over the block's MFMA slots
      if constexpr (kCopy) {
#pragma unroll
        for (int i = 0; i < kCopies; ++i)
          if (t == i * kMfmas / kCopies) copy_one(*cp, i);
      }
      // Probabilities of the 8 score pairs, software-pipelined so that each
      // step of a pair (scale, exp2, then pack and fp32 partial sum) runs a
      // few MFMA slots after the step it depends on and never stalls the
      // wave's in-order issue.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (t == slot(e, 0)) {
          pr[2 * e] = __builtin_fmaf(s_cur[2 * e], c, neg_mc);
          pr[2 * e + 1] = __builtin_fmaf(s_cur[2 * e + 1], c, neg_mc);
        }
        if (t == slot(e, 1)) {
          pr[2 * e] = __builtin_amdgcn_exp2f(pr[2 * e]);
          pr[2 * e + 1] = __builtin_amdgcn_exp2f(pr[2 * e + 1]);
        }
        if (t == slot(e, 2)) {
          pw[e >> 2][e & 3] = E::pack2(pr[2 * e], pr[2 * e + 1]);
          const float pair = pr[2 * e] + pr[2 * e + 1];
          sum[e & 1] = e < 2 ? pair : sum[e & 1] + pair;
        }
      }
      // half way through the block the wave's priority steps down
      if (t == kMfmas / 2 - 1) __builtin_amdgcn_s_setprio(kHalf == 0 ? 2 : 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Keep the packing inside the MFMA stream: the reference-update path below
    // overwrites pw, and without this use the compiler sinks the conversions
    // past its branch, right in front of the next block's first PV MFMA.
    asm volatile("" ::"v"(pw[0]), "v"(pw[1]));
    float s_tot = sum[0] + sum[1];
    if (!kFirst && __builtin_amdgcn_ballot_w64(s_tot > kSumCap<IsBf16>) != 0) {
      // rare: some probability of this block may exceed the cap (or a row
      // sees its first key).  The scores are formed again from LDS rather
      // than kept live through the block.
      const f32x16 st = scores<kMask>(u);
      raise_reference(st);
      s_tot = 0.f;
      float s2 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) exp_pair(st, e, pw, (e & 1) ? s2 : s_tot);
      s_tot += s2;
    }
    l_part += s_tot;
    p_prev[0] = pw[0];
    p_prev[1] = pw[1];
    s_cur = s_next;
    if (kHalf == 0) __builtin_amdgcn_s_setprio(1);
  }

  // PV MFMAs of the wave's last block.
  __device__ __forceinline__ void drain() {
#pragma unroll
    for (int t = 0; t < kPV; ++t)
      acc[t >> 1] = E::mfma(vfr[t], __builtin_bit_cast(vec8, p_prev[t & 1]), acc[t >> 1]);
  }

  // Tile step j: blocks 2j and 2j+1.  They read K tiles j (second half) and
  // j+1 (first half) and V tile j.  The step copies K tile j+3 (into the stage
  // K tile j-1 left) and V tile j+2 (into the stage V tile j-2 left) and,
  // before its closing barrier, waits only for the copies issued one step
  // earlier, so every copy has two steps to land.
  //
  // In the workgroup's first step (kFirstStep) a wave whose first block u_lo
  // lies in the step runs it as kFirst; u_lo is never below 2j there.
  //
  // Issue priority.  The two waves of a SIMD run the same code, and with equal
  // priorities the older one always issues first: it reaches the barrier well
  // ahead and idles while the other finishes the step alone, without a second
  // wave to overlap its MFMAs and VALU work.  So a wave's priority falls as it
  // gets through the step (3 at the start, 2, 1, 0 at each half block): the
  // wave that is behind issues first and the pair stays level.
  template <int kMask, bool kFirstStep = false>
  __device__ __forceinline__ void step(int j) {
    __builtin_amdgcn_s_setprio(3);
    // block 2j spreads the step's copies over its MFMAs, so that the texture
    // unit moves them while the matrix cores work; a wave that does not
    // compute that block issues them at once
    const Copies cp = prepare_tiles(j + 3, (j + 3) & 3, j + 2, (j + 2) & 3);
    if (kFirstStep) {
#pragma unroll
      for (int i = 0; i < kCopies; ++i) copy_one(cp, i);
      if (u_lo == 2 * j && u_lo < n_sub) block<kMask, true, 0>(2 * j);
      if (u_lo == 2 * j + 1 && u_lo < n_sub)
        block<kMask, true, 1>(2 * j + 1);
      else if (u_lo == 2 * j && 2 * j + 1 < n_sub)
        block<kMask, false, 1>(2 * j + 1);
    } else {
      const int u = 2 * j;
      if (u >= u_lo && u < n_sub) {
        block<kMask, false, 0, true>(u, &cp);
      } else {
#pragma unroll
        for (int i = 0; i < kCopies; ++i) copy_one(cp, i);
      }
      if (u + 1 >= u_lo && u + 1 < n_sub) block<kMask, false, 1>(u + 1);
    }
    __builtin_amdgcn_s_setprio(0);
    wait_older_copies();
    __syncthreads();
  }

  // Whether this wave's 64-row query block sees the tile at list position p
  // (wave-uniform).
  __device__ __forceinline__ bool sees(int p) const {
    return p < n_pos && q0 < N &&
           ((__builtin_amdgcn_readfirstlane((int)tiles[p]) >> qbit) & 1) != 0;
  }

  // Block-sparse tile step j (list position j).  A wave computes the two
  // blocks of the tile only if its query block sees it, so each wave walks
  // runs of visible positions and sits out the rest.  A run's first block
  // forms its own scores from the resident K tile (the prefetched ones belong
  // to a hidden block); its PV MFMAs are those the previous run's last block
  // left pending (zeros before the first run), so nothing is drained between
  // runs.  A row without a reference yet (kNoRef) takes the block's
  // reference-update path.  A visible tile needs no block mask, only the
  // causal and sequence-end masks.  The copies and the barrier are the
  // workgroup's, as in step().
  __device__ __forceinline__ void sparse_step(int j) {
    __builtin_amdgcn_s_setprio(3);
    load_tiles(tile_at(j + 3), (j + 3) & 3, tile_at(j + 2), (j + 2) & 3);
    const bool vis = sees(j);
    if (vis) {
      if (!live) s_cur = scores<kMaskNone>(2 * j);
      block<kMaskEdge, false, 0>(2 * j);
      block<kMaskEdge, false, 1>(2 * j + 1);
    }
    live = vis;
    __builtin_amdgcn_s_setprio(0);
    wait_older_copies();
    __syncthreads();
  }

  // LDS holds rings of kStages K tiles and kStages V tiles; tile j lives in
  // stage j & 3.  The workgroup's first tile j_lo is the first one that any of
  // its queries can see (0 unless a sliding window starts later).
  // Block-sparse: list the key tiles that some query block of this workgroup
  // may see (the causal limit included), in order, each with one bit per
  // 64-row query block; rows of the mask past N read as hidden.
  __device__ __forceinline__ void build_tile_list(uint32_t* list, const uint8_t* mask, int q0_blk) {
    const int n_kb = (N + kBN - 1) / kBN, n_qb = (N + kSparseBlock - 1) / kSparseBlock;
    const int qb0 = q0_blk / kSparseBlock;
    const int nt = n_tiles;
    n_pos = compact_tiles<kWaves>(list, nt, [&](int jt) {
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < kBM / kSparseBlock; ++i) {
        const int qb = qb0 + i;
        if (qb < n_qb && (!Causal || jt <= qb) && mask[(int64_t)qb * n_kb + jt] != 0) bits |= 1u << i;
      }
      return bits;
    });
  }

  __device__ __forceinline__ void run(int q0_blk, uint32_t* list = nullptr, const uint8_t* mask = nullptr) {
    static_assert(kStages == 4, "the ring arithmetic assumes four stages");
    if constexpr (kSparse) {
      build_tile_list(list, mask, q0_blk);
      tiles = list;
      // prologue as below, by list position
      load_tiles(tile_at(0), 0, tile_at(0), 0);
      load_tiles(tile_at(1), 1, tile_at(1), 1);
      load_tiles(tile_at(2), 2, n_tiles, 3);
      wait_older_copies();
      __syncthreads();
      live = false;
      for (int j = 0; j < n_pos; ++j) sparse_step(j);
      drain();  // the last run's last block (adds 0 if the wave saw nothing)
      return;
    }
    const int j_lo = kWin ? max(0, q0_blk - win + 1) / kBN : 0;
    // prologue: K, V tiles j_lo, j_lo+1 resident; K tile j_lo+2 in flight (its
    // V slot copies zeros into the stage V tile j_lo+3 overwrites one step later)
    load_tiles(j_lo, j_lo & 3, j_lo, j_lo & 3);
    load_tiles(j_lo + 1, (j_lo + 1) & 3, j_lo + 1, (j_lo + 1) & 3);
    load_tiles(j_lo + 2, (j_lo + 2) & 3, n_tiles, (j_lo + 3) & 3);
    wait_older_copies();
    __syncthreads();
    // scores of the first block of every wave that starts in the first step
    // (all of them without a sliding window); K tile j_lo is resident
    if (u_lo < 2 * j_lo + 2 && u_lo < n_sub) s_cur = scores<kMaskNone>(u_lo);

    // Steps that may need a mask: those before j_left (some query's window
    // starts inside one of their blocks) and from j_mask on (causal diagonal
    // or the end of the sequence).
    const int u_left = kWin ? (max(0, q0_blk + kBM - win) + 31) / 32 : 0;
    const int j_left = (u_left + 1) / 2;
    const int u_mask = Causal ? q0_blk / 32 : ((N % 32) ? N / 32 : (N + 31) / 32 + 2);
    const int j_mask = max(j_left, u_mask / 2);
    step<kMaskWindow, true>(j_lo);
    int j = j_lo + 1;
    for (; j < min(j_left, n_tiles); ++j) step<kMaskWindow>(j);
    for (; j < min(j_mask, n_tiles); ++j) step<kMaskNone>(j);
    for (; j < n_tiles; ++j) step<kMaskEdge>(j);
    if (n_sub > u_lo) drain();
  }

  // O = a / l once; LSE = ln(sum) of the scaled scores.  Block-sparse rows
  // that see no key store O = 0 and LSE = -inf.
  __device__ __forceinline__ void store(uint16_t* O, float* LSE, int bh) {
    if (!kSparse && n_sub <= u_lo) return;
    const float l_tot = xhalf_sum(l_part);
    const float inv = (!kSparse || l_tot > 0.f) ? 1.0f / l_tot : 0.f;
    if (my_q >= N) return;
    uint16_t* orow = O + o_off + (int64_t)my_q * o_sn;
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

template <bool IsBf16, int D, bool Causal, int Mode, int DV>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int win, int H, int BH, int n_qblocks,
    float c, uint32_t q_sign, Layout lq, Layout in, Layout lv, Layout out,
    const uint8_t* __restrict__ bmask, int64_t m_sb, int64_t m_sh) {
  using L = Lds<D, DV>;
  static_assert(L::kBytes + kSparseBytes <= 160 * 1024, "the tile list fits beside the rings");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::kBytes + (Mode == kModeSparse ? kSparseBytes : 0)];
  // work item: (query block, batch*head); heaviest causal blocks first
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (Causal) qb = n_qblocks - 1 - qb;
  FwdBlock<IsBf16, D, Causal, Mode, DV> blk;
  blk.init(smem, Q, K, V, N, win, H, bh, qb, c, q_sign, lq, in, lv, out);
  if constexpr (Mode == kModeSparse) {
    const int b = bh / H, h = bh - b * H;
    blk.qbit = 16 + blk.wave / 2;  // 32-row waves, 64-row mask blocks
    blk.run(qb * kBM, reinterpret_cast<uint32_t*>(smem + L::kBytes), bmask + b * m_sb + h * m_sh);
  } else {
    blk.run(qb * kBM);
  }
  blk.store(O, LSE, bh);
}

template <bool IsBf16, int D, bool Causal, int Mode, int DV = D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int N = (int)a.N;
  const int BH = (int)(a.B * a.H);
  int n_qblocks = (N + kBM - 1) / kBM;
  // Unmasked, with a last query block of at most 32 rows: that block would
  // stream every key through one wave in a round of its own, so the tail
  // kernel takes those rows with the keys split over its waves.
  if (!Causal && Mode == kModePlain && DV == D && N % kBM != 0 && N % kBM <= 32) {
    n_qblocks -= 1;
    const hipError_t e = IsBf16 ? launch_fwd_tail_bf16(a, (int64_t)n_qblocks * kBM, stream)
                                : launch_fwd_tail_f16(a, (int64_t)n_qblocks * kBM, stream);
    if (e != hipSuccess || n_qblocks == 0) return e;
  }
  const dim3 grid((unsigned)(n_qblocks * BH));
  // c = |scale| * log2(e).  A zero scale is run as the limit scale -> 0+:
  // with c = 1e-30 every exp2 argument c*(s - m) rounds to exactly 0 in fp32,
  // so all visible keys weigh exactly 1 and hidden ones (-inf) weigh 0.
  const float c = a.scale != 0.f ? __builtin_fabsf(a.scale) * 1.4426950408889634f : 1e-30f;
  const uint32_t q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<IsBf16, D, Causal, Mode, DV>), grid, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, N,
                     (int)(a.window < a.N ? a.window : a.N), (int)a.H, BH, n_qblocks, c, q_sign, a.lq,
                     a.in, a.lv, a.out, a.block_mask, a.mask_sb, a.mask_sh);
  return hipGetLastError();
}

template <bool IsBf16, int D>
hipError_t dispatch_d(const FwdArgs& a, hipStream_t s) {
  if (a.block_mask != nullptr)
    return a.causal ? launch<IsBf16, D, true, kModeSparse>(a, s) : launch<IsBf16, D, false, kModeSparse>(a, s);
  if (!a.causal) return launch<IsBf16, D, false, kModePlain>(a, s);
  if (a.window < a.N) return launch<IsBf16, D, true, kModeWindow>(a, s);
  return launch<IsBf16, D, true, kModePlain>(a, s);
}

}  // namespace

hipError_t launch_fwd64_bf16(const FwdArgs& a, hipStream_t s) { return dispatch_d<true, 64>(a, s); }
hipError_t launch_fwd64_f16(const FwdArgs& a, hipStream_t s) { return dispatch_d<false, 64>(a, s); }

}  // namespace fa
