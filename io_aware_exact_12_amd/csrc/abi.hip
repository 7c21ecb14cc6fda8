// C ABI of libfa_attn.so: argument validation, kernel choice and launch.
// The declarations and their contract are in include/fa_attn.h.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_attn.h"
#include "fa_internal.hpp"

namespace {

constexpr int kAbiVersion = 11;
// Block-sparse: mask blocks of 64 x 64; a query block of the forward lists at
// most this many key tiles (its LDS list).
constexpr int64_t kMaxSparseTiles = 2048;
// Largest query-block count times B*H that still indexes a 1-D grid, with the
// smallest query block any kernel uses (64 rows).
constexpr int64_t kMaxGrid = (int64_t)INT32_MAX;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the forward and backward entry points.
int check_common(int64_t B, int64_t H, int64_t N, int64_t d, int mask, float scale, int dtype) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_SHAPE;
  if (N > INT32_MAX / 2 || B > INT32_MAX || H > INT32_MAX) return FA_ERR_SHAPE;
  if (B * H > INT32_MAX) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh > INT64_MAX / N || bh * N > INT64_MAX / 128 / 4) return FA_ERR_SHAPE;
  if (((N + 63) / 64) * bh > kMaxGrid) return FA_ERR_SHAPE;
  if (d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  // one head of a dense [N][d] array must span less than 2 GiB (one buffer resource)
  if (N * d * (dtype == FA_F32 ? 4 : 2) > INT32_MAX - 1024) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

size_t elt_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// A strided view ([B][H][N][d], d contiguous, strides {batch, head, row} in
// elements) is usable when every stride is >= 0 and a multiple of 16 bytes,
// rows are at least d elements apart, and one head's rows span less than
// 2 GiB (the kernels address a head through one buffer resource).  Outputs
// must in addition not overlap: ordered by stride, each dimension of extent
// > 1 must step past everything the smaller ones cover.
int check_layout(const int64_t* st, int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                 bool output, fa::Layout* out) {
  if (st == nullptr) return FA_ERR_NULL;
  const int64_t align = 16 / (int64_t)elt_bytes(dtype);
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % align != 0 || st[i] > INT64_MAX / 4 / (i == 0 ? B : i == 1 ? H : N))
      return FA_ERR_STRIDE;
  if (st[2] < d) return FA_ERR_STRIDE;
  if ((N - 1) * st[2] > (INT32_MAX - 1024) / (int64_t)elt_bytes(dtype) - d) return FA_ERR_SHAPE;
  if (output) {
    int64_t cnt[3] = {B, H, N}, str[3] = {st[0], st[1], st[2]};
    for (int i = 0; i < 3; ++i)  // order by stride
      for (int j = i + 1; j < 3; ++j)
        if (str[j] < str[i]) {
          const int64_t a = str[i], c = cnt[i];
          str[i] = str[j], cnt[i] = cnt[j], str[j] = a, cnt[j] = c;
        }
    int64_t ext = d;
    for (int i = 0; i < 3; ++i) {
      if (cnt[i] == 1) continue;
      if (str[i] < ext) return FA_ERR_STRIDE;
      ext += (cnt[i] - 1) * str[i];
    }
  }
  *out = fa::Layout{st[0], st[1], st[2]};
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
             int64_t N, int64_t d, int mask, int64_t window, float scale, int dtype, void* stream,
             const int64_t* q_st = nullptr, const int64_t* kv_st = nullptr,
             const int64_t* out_st = nullptr, const uint8_t* block_mask = nullptr,
             int64_t mask_b = 0, int64_t mask_h = 0, int64_t dv = 0) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_NULL;
  const int st = check_common(B, H, N, d, mask, scale, dtype);
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, mask == FA_MASK_CAUSAL, scale, window < N ? window : N,
                fa::dense_layout(H, N, d), fa::dense_layout(H, N, d), fa::dense_layout(H, N, d)};
  a.dv = d;
  if (dv != 0 && dv != d) {  // v and o rows of dv elements, dense
    if (!fa::dv_pair_built(d, dv)) return FA_ERR_UNSUPPORTED;
    a.dv = dv;
    a.out = fa::dense_layout(H, N, dv);
  }
  if (q_st != nullptr || kv_st != nullptr || out_st != nullptr) {
    int e1 = check_layout(q_st, B, H, N, d, dtype, false, &a.lq);
    if (e1 == FA_OK) e1 = check_layout(kv_st, B, H, N, d, dtype, false, &a.in);
    if (e1 == FA_OK) e1 = check_layout(out_st, B, H, N, d, dtype, true, &a.out);
    if (e1 != FA_OK) return e1;
  }
  if (block_mask != nullptr) {
    const int64_t nb = (N + 63) / 64;
    if ((mask_b != 1 && mask_b != B) || (mask_h != 1 && mask_h != H)) return FA_ERR_SHAPE;
    if (nb > kMaxSparseTiles) return FA_ERR_UNSUPPORTED;
    a.block_mask = block_mask;
    a.mask_sh = mask_h == 1 ? 0 : nb * nb;
    a.mask_sb = mask_b == 1 ? 0 : mask_h * nb * nb;
  }
  a.lv = a.dv == d ? a.in : fa::dense_layout(H, N, a.dv);
  // d = 256 or d_v = 256: bf16 / fp16 (the wide kernel)
  const bool wide = d == 256 || a.dv == 256;
  if (wide && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return FA_ERR_ALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (wide) {
    e = dtype == FA_BF16 ? fa::launch_fwd_wide_bf16(a, s) : fa::launch_fwd_wide_f16(a, s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  switch (dtype) {
    case FA_BF16: e = fa::launch_fwd_bf16(a, s); break;
    case FA_F16: e = fa::launch_fwd_f16(a, s); break;
    default: e = fa::launch_fwd_f32(a, s); break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
             int64_t d, int mask, int64_t window, float scale, int dtype, void* workspace,
             size_t workspace_bytes, void* stream, const int64_t* in_st = nullptr,
             const int64_t* out_st = nullptr, const uint8_t* block_mask = nullptr,
             int64_t mask_b = 0, int64_t mask_h = 0, int64_t dvw = 0) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr ||
      lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return FA_ERR_NULL;
  const int st = check_common(B, H, N, d, mask, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  const size_t need = block_mask != nullptr ? fa::bwd_sparse_workspace_bytes(B, H, N, d)
                                            : fa::bwd_workspace_bytes(B, H, N);
  if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask == FA_MASK_CAUSAL, scale,
                workspace, window < N ? window : N, fa::dense_layout(H, N, d),
                fa::dense_layout(H, N, d)};
  if (in_st != nullptr || out_st != nullptr) {
    int e1 = check_layout(in_st, B, H, N, d, dtype, false, &a.in);
    if (e1 != FA_OK) return e1;
    e1 = check_layout(out_st, B, H, N, d, dtype, true, &a.out);
    if (e1 != FA_OK) return e1;
  }
  if (block_mask != nullptr) {
    const int64_t nb = (N + 63) / 64;
    if ((mask_b != 1 && mask_b != B) || (mask_h != 1 && mask_h != H)) return FA_ERR_SHAPE;
    if (nb > kMaxSparseTiles) return FA_ERR_UNSUPPORTED;
    // the dK/dV grid: up to kBwdSparseSplit workgroups per 128-key block and head
    if (((N + 127) / 128) * B * H > kMaxGrid / fa::kBwdSparseSplit) return FA_ERR_SHAPE;
    a.block_mask = block_mask;
    a.mask_sh = mask_h == 1 ? 0 : nb * nb;
    a.mask_sb = mask_b == 1 ? 0 : mask_h * nb * nb;
  }
  a.dvw = d;
  a.lv = a.in;
  a.outv = a.out;
  if (dvw != 0 && dvw != d) {  // v, o, dout and dv rows of dvw elements, dense
    if (!fa::dv_pair_built(d, dvw)) return FA_ERR_UNSUPPORTED;
    a.dvw = dvw;
    a.lv = a.outv = fa::dense_layout(H, N, dvw);
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return FA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_BF16 ? fa::launch_bwd_bf16(a, s) : fa::launch_bwd_f16(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int kv_outer_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                  int64_t H, int64_t N, int64_t d, int mask, float scale, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_NULL;
  const int st = check_common(B, H, N, d, mask, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32 || d == 256) return FA_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < fa::kv_outer_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, mask == FA_MASK_CAUSAL, scale, N,
                fa::dense_layout(H, N, d), fa::dense_layout(H, N, d), fa::dense_layout(H, N, d)};
  a.dv = d;
  a.lv = a.in;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_kv_outer_bf16(a, workspace, s)
                                        : fa::launch_fwd_kv_outer_f16(a, workspace, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------- allocation-free backward
// attn_bwd_noalloc takes its scratch (the backward's two fp32 terms per query
// row, fa::bwd_workspace_bytes) from this fixed array instead of a caller
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends; calls on one GPU share it, so calls that overlap in time on
// one GPU race on it.
constexpr size_t kScratchBytes = (size_t)8 << 20;  // B * H * N <= 1,048,576 query rows
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept.  In host code the array's name
// is only a host-side stand-in: kernels get this address, never the name.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
             int64_t H, int64_t N, int64_t d, int mask, float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, mask, N, scale, dtype, stream);
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                    int64_t H, int64_t N, int64_t d, int64_t window, float scale, int dtype,
                    void* stream) {
  if (window < 1) return FA_ERR_WINDOW;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, FA_MASK_CAUSAL, window, scale, dtype, stream);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (check_common(B, H, N, d, FA_MASK_NONE, 1.0f, dtype) != FA_OK) return 0;
  return fa::bwd_workspace_bytes(B, H, N);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
             int64_t d, int mask, float scale, int dtype, void* workspace, size_t workspace_bytes,
             void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, N, scale, dtype, workspace,
                  workspace_bytes, stream);
}

size_t attn_bwd_noalloc_max_rows(void) { return kScratchBytes / 8; }

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                     int64_t d, int mask, float scale, int dtype, void* stream) {
  // the shape checks bound B * H * N before the scratch size is formed
  const int st = check_common(B, H, N, d, mask, scale, dtype);
  if (st != FA_OK) return st;
  if (fa::bwd_workspace_bytes(B, H, N) > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  const int e = scratch_of_current_device(&ws);
  if (e != FA_OK) return e;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, N, scale, dtype, ws,
                  kScratchBytes, stream);
}

int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                    int64_t d, int64_t window, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (window < 1) return FA_ERR_WINDOW;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, FA_MASK_CAUSAL, window, scale, dtype,
                  workspace, workspace_bytes, stream);
}

int attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t N, int64_t d, const int64_t* q_strides,
                     const int64_t* kv_strides, const int64_t* o_strides, int mask, float scale,
                     int dtype, void* stream) {
  if (q_strides == nullptr || kv_strides == nullptr || o_strides == nullptr) return FA_ERR_NULL;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, mask, N, scale, dtype, stream, q_strides, kv_strides,
                  o_strides);
}

int attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                     int64_t d, const int64_t* in_strides, const int64_t* grad_strides, int mask,
                     float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (in_strides == nullptr || grad_strides == nullptr) return FA_ERR_NULL;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, N, scale, dtype, workspace,
                  workspace_bytes, stream, in_strides, grad_strides);
}

int attn_fwd_dv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t H, int64_t N, int64_t d, int64_t dv, int mask, float scale, int dtype,
                void* stream) {
  if (dv < 1) return FA_ERR_SHAPE;
  if (dv != 64 && dv != 96 && dv != 128 && dv != 256) return FA_ERR_UNSUPPORTED;
  // bound N first: N * dv * 4 then cannot overflow int64
  if (N > 0 && (N > INT32_MAX / 2 || N * dv * (dtype == FA_F32 ? 4 : 2) > INT32_MAX - 1024))
    return FA_ERR_SHAPE;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, mask, N, scale, dtype, stream, nullptr, nullptr,
                  nullptr, nullptr, 0, 0, dv);
}

int attn_bwd_dv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                int64_t d, int64_t d_v, int mask, float scale, int dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (d_v < 1) return FA_ERR_SHAPE;
  if (d_v != 64 && d_v != 96 && d_v != 128 && d_v != 256) return FA_ERR_UNSUPPORTED;
  // bound N first: N * d_v * 4 then cannot overflow int64
  if (N > 0 && (N > INT32_MAX / 2 || N * d_v * (dtype == FA_F32 ? 4 : 2) > INT32_MAX - 1024))
    return FA_ERR_SHAPE;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, N, scale, dtype, workspace,
                  workspace_bytes, stream, nullptr, nullptr, nullptr, 0, 0, d_v);
}

int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t d, const uint8_t* block_mask,
                          int64_t mask_batches, int64_t mask_heads, int mask, float scale, int dtype,
                          void* stream) {
  if (block_mask == nullptr) return FA_ERR_NULL;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, mask, N, scale, dtype, stream, nullptr, nullptr,
                  nullptr, block_mask, mask_batches, mask_heads);
}

size_t attn_bwd_block_sparse_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (check_common(B, H, N, d, FA_MASK_NONE, 1.0f, dtype) != FA_OK) return 0;
  return fa::bwd_sparse_workspace_bytes(B, H, N, d);
}

int attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv, int64_t B,
                          int64_t H, int64_t N, int64_t d, const uint8_t* block_mask,
                          int64_t mask_batches, int64_t mask_heads, int mask, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (block_mask == nullptr) return FA_ERR_NULL;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask, N, scale, dtype, workspace,
                  workspace_bytes, stream, nullptr, nullptr, block_mask, mask_batches, mask_heads);
}

size_t attn_fwd_kv_outer_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (check_common(B, H, N, d, FA_MASK_NONE, 1.0f, dtype) != FA_OK || dtype == FA_F32 || d == 256)
    return 0;
  return fa::kv_outer_workspace_bytes(B, H, N, d);
}

int attn_fwd_kv_outer(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t H, int64_t N, int64_t d, int mask, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return kv_outer_impl(q, k, v, o, lse, B, H, N, d, mask, scale, dtype, workspace, workspace_bytes,
                       stream);
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is < 1 or the problem is too large to index";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_MASK: return "unknown mask";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_UNSUPPORTED:
      return "unsupported: head dimension must be 64, 96, 128 or 256 (256: fp16/bf16 and plain, "
             "strided, window or block-sparse calls only), d_v must be d or (d, d_v) in {(128, 64), "
             "(64, 128)}; the backward and the key/value-outer forward take fp16/bf16 only";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "the HIP runtime rejected a launch";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_WINDOW: return "sliding window must be >= 1";
    case FA_ERR_STRIDE: return "a stride is negative, not a multiple of 16 bytes, below d (rows), or makes output rows overlap";
    case FA_ERR_SCRATCH:
      return "B * H * N exceeds the fixed scratch of the allocation-free backward "
             "(attn_bwd_noalloc_max_rows() query rows)";
    default: return "unknown status";
  }
}

int fa_abi_version(void) { return kAbiVersion; }

}  // extern "C"
