// Internal declarations shared by the launch code of libfa_attn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {

// Element strides of a [B][H][N][d] view whose d axis is contiguous: batch,
// head and row.  A dense [B][H][N][d] array has {H*N*d, N*d, d}; a
// [B][N][H][d] one {N*H*d, d, H*d}.
struct Layout {
  int64_t sb, sh, sn;
};

inline Layout dense_layout(int64_t H, int64_t N, int64_t d) { return Layout{H * N * d, N * d, d}; }

// Arguments of one forward launch after validation.  Pointers are device
// pointers to [B][H][N][d] views with layouts `lq` (q), `in` (k and v) and
// `out` (o); lse is a dense [B][H][N] array (may be null).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t B, H, N, d;
  bool causal;
  float scale;
  // causal only: key j is visible to query i iff i - window < j <= i
  // (window >= N is plain causal)
  int64_t window;
  Layout lq, in, out;
  // block-sparse mask (or null): uint8 [mask batch][mask head][ceil(N/64)][ceil(N/64)]
  // with element strides mask_sb, mask_sh (0 broadcasts over batch or head)
  const uint8_t* block_mask;
  int64_t mask_sb, mask_sh;
  // width of v and o rows (d_v; equal to d except in the d_v != d call) and v's layout
  int64_t dv;
  Layout lv;
};

// Arguments of one backward launch after validation.  workspace holds at
// least bwd_workspace_bytes(B, H, N) bytes of device memory.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t B, H, N, d;
  bool causal;
  float scale;
  void* workspace;
  int64_t window;  // as for FwdArgs
  Layout in;       // q, k, v, o, dout
  Layout out;      // dq, dk, dv
  const uint8_t* block_mask;  // as for FwdArgs
  int64_t mask_sb, mask_sh;
  int64_t dvw;     // width of v, o, dout, dv rows (d_v; d except in the d_v != d call)
  Layout lv;       // v, o, dout
  Layout outv;     // dv
};

// The block-sparse backward cuts a key block's list of query tiles into at
// most this many chunks, each run by a dK/dV workgroup of its own.
constexpr int kBwdSparseSplit = 4;

// Widths of v (and o, dout, dv) rows other than d that the kernels are built
// for: d and d_v in {64, 96, 128, 256}, d_v != d.  A pair with a 256 side runs
// the d = 256 kernels (bf16 / fp16 only); the others run the MFMA kernels of
// d <= 128 and the fp32 path.
inline bool dv_pair_built(int64_t d, int64_t dv) {
  auto ok = [](int64_t x) { return x == 64 || x == 96 || x == 128 || x == 256; };
  return ok(d) && ok(dv) && d != dv;
}

// Launchers return the hipError_t of the launch (hipSuccess when enqueued).
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t s);
// d = d_v = 64 (fwd_mfma64.hip)
hipError_t launch_fwd64_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd64_f16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
// Tail rows r0 .. N-1 (at most 32) of an unmasked bf16 / fp16 forward with
// d_v = d in {64, 96, 128}: one workgroup per head, keys split over its waves.
hipError_t launch_fwd_tail_bf16(const FwdArgs& a, int64_t r0, hipStream_t s);
hipError_t launch_fwd_tail_f16(const FwdArgs& a, int64_t r0, hipStream_t s);
// d = 256 forward (plain masks, d_v = d): one 4-wave workgroup per CU
hipError_t launch_fwd_wide_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_wide_f16(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_f16(const BwdArgs& a, hipStream_t s);
size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N);
// Block-sparse backward: also chunk counters and fp32 partial dK, dV of up to
// four chunks of every key's query-tile list.
size_t bwd_sparse_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);
// Key/value-outer forward (the comparison loop order): fp32 row state
// (O, m, l) of B*H*N rows in ws.
hipError_t launch_fwd_kv_outer_bf16(const FwdArgs& a, void* ws, hipStream_t s);
hipError_t launch_fwd_kv_outer_f16(const FwdArgs& a, void* ws, hipStream_t s);
size_t kv_outer_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

}  // namespace fa
