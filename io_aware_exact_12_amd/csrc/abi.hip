// C ABI of libfa_attn.so: argument validation, kernel choice and launch.
// The declarations and their contract are in include/fa_attn.h.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "fa_attn.h"
#include "fa_internal.hpp"

namespace {

constexpr int kAbiVersion = 3;
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
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
             int64_t N, int64_t d, int mask, int64_t window, float scale, int dtype, void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_NULL;
  const int st = check_common(B, H, N, d, mask, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return FA_ERR_ALIGN;

  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, mask == FA_MASK_CAUSAL, scale, window < N ? window : N};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
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
             size_t workspace_bytes, void* stream) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr ||
      lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return FA_ERR_NULL;
  const int st = check_common(B, H, N, d, mask, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < fa::bwd_workspace_bytes(B, H, N))
    return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return FA_ERR_ALIGN;
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, mask == FA_MASK_CAUSAL, scale,
                workspace, window < N ? window : N};
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
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < fa::kv_outer_workspace_bytes(B, H, N, d))
    return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, mask == FA_MASK_CAUSAL, scale, N};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_kv_outer_bf16(a, workspace, s)
                                        : fa::launch_fwd_kv_outer_f16(a, workspace, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
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

int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                    int64_t d, int64_t window, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (window < 1) return FA_ERR_WINDOW;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, FA_MASK_CAUSAL, window, scale, dtype,
                  workspace, workspace_bytes, stream);
}

size_t attn_fwd_kv_outer_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (check_common(B, H, N, d, FA_MASK_NONE, 1.0f, dtype) != FA_OK || dtype == FA_F32) return 0;
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
    case FA_ERR_UNSUPPORTED: return "unsupported: head dimension must be 64 or 128 (backward: fp16/bf16 only)";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "the HIP runtime rejected a launch";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_WINDOW: return "sliding window must be >= 1";
    default: return "unknown status";
  }
}

int fa_abi_version(void) { return kAbiVersion; }

}  // extern "C"
