// C ABI of the attention library: host-side validation, then dispatch to the kernel files.
// Every check runs before any HIP call, so invalid arguments never reach the GPU.
#include "fa.h"

#include <cmath>
#include <cstdint>

#include "fa_launch.h"

static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_SCRATCH_BYTES, "scratch size in fa.h and fa_launch.h");

namespace {

constexpr int64_t kI32Max = 2147483647;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool dtype_ok(fa_dtype_t t) { return t == FA_DTYPE_BF16 || t == FA_DTYPE_F32; }
int64_t elt_bytes(fa_dtype_t t) { return t == FA_DTYPE_BF16 ? 2 : 4; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }
// One head's tensor must be addressable with 32-bit byte offsets.
bool head_fits(int64_t n, int64_t d, fa_dtype_t t) { return n <= kI32Max / (d * elt_bytes(t)); }

fa_status_t from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// The forward behind fa_fwd and fa_fwd_ex; `mask` already known to be one of the three values.
// square_causal: fa_fwd's contract, a causal mask only with Nq == Nk.
fa_status_t forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                    int64_t H_kv, int64_t Nq, int64_t Nk, int64_t d, fa_mask_t mask, bool square_causal,
                    float scale, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!dtype_ok(dtype) || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  if (B <= 0 || H <= 0 || H_kv <= 0 || Nq <= 0 || Nk <= 0 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (mask == FA_MASK_CAUSAL_BOTTOM_RIGHT && Nk < Nq) return FA_ERR_SHAPE;  // a row would see no key
  if (square_causal && mask != FA_MASK_NONE && Nq != Nk) return FA_ERR_SHAPE;
  if (!head_fits(Nq, d, dtype) || !head_fits(Nk, d, dtype)) return FA_ERR_SHAPE;
  if (B > kI32Max / H || B * H > kI32Max / ((Nq + 31) / 32)) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_ARG;
  int dev = 0, num_cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || num_cus <= 0)
    return FA_ERR_HIP;
  const bool causal = mask != FA_MASK_NONE;
  const int diag = mask == FA_MASK_CAUSAL_BOTTOM_RIGHT ? (int)(Nk - Nq) : 0;
  fa::FwdArgs a{q, k, v, o, lse, (int)B, (int)H, (int)Nq, (int)Nk, (int)d, (int)H_kv, causal, diag, scale, num_cus};
  return from_hip(dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(a, stream) : fa::launch_fwd_f32(a, stream));
}

// The split step behind fa_decode_split and fa_decode_split_ex.
fa_status_t decode_split(const void* q, const void* k, const void* v, void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t H, int64_t H_kv, int64_t Nk, int64_t d, float scale, int num_splits,
                         fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !workspace) return FA_ERR_NULL;
  if (!dtype_ok(dtype) || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(workspace, 16)) return FA_ERR_ALIGN;
  if (B <= 0 || H <= 0 || H_kv <= 0 || Nk <= 0 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (!head_fits(Nk, d, dtype) || B > kI32Max / H) return FA_ERR_SHAPE;
  if (num_splits < 1 || num_splits > Nk || !scale_ok(scale)) return FA_ERR_ARG;
  if (B * H > kI32Max / num_splits) return FA_ERR_SHAPE;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  float* o_part = static_cast<float*>(workspace);
  float* ml = o_part + (size_t)(B * H * num_splits) * (size_t)d;
  fa::DecodeSplitArgs a{q, k, v, o_part, ml, (int)B, (int)H, (int)Nk, (int)d, num_splits, (int)H_kv, scale};
  return from_hip(dtype == FA_DTYPE_BF16 ? fa::launch_decode_split_bf16(a, stream)
                                         : fa::launch_decode_split_f32(a, stream));
}

// Masked-forward workspace: tile counts (int32 per query block), tile classes (a byte per block
// and tile), tile lists (uint16 per block and tile) and the forward's claim counter (16 bytes), each
// part starting on 16 bytes.
int64_t mask_ws_counts_bytes(int64_t n_qblk) { return (4 * n_qblk + 15) / 16 * 16; }
int64_t mask_ws_cls_bytes(int64_t n_qblk, int64_t nT) { return (n_qblk * nT + 15) / 16 * 16; }
int64_t mask_ws_lists_bytes(int64_t n_qblk, int64_t nT) { return (2 * n_qblk * nT + 15) / 16 * 16; }

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, fa_dtype_t dtype,
                   hipStream_t stream) {
  return forward(q, k, v, o, lse, B, H, H, Nq, Nk, d, causal ? FA_MASK_CAUSAL : FA_MASK_NONE, true, scale, dtype,
                 stream);
}

fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                      int64_t H_kv, int64_t Nq, int64_t Nk, int64_t d, fa_mask_t mask, float scale, fa_dtype_t dtype,
                      hipStream_t stream) {
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_CAUSAL_BOTTOM_RIGHT) return FA_ERR_ARG;
  return forward(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, mask, false, scale, dtype, stream);
}

fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_scale, const float* k_scale,
                       const float* v_scale, void* o, float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t Nq,
                       int64_t Nk, int64_t d, fa_mask_t mask, float scale, hipStream_t stream) {
  if (!q || !k || !v || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_NULL;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_CAUSAL_BOTTOM_RIGHT) return FA_ERR_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return FA_ERR_ALIGN;
  if (B <= 0 || H <= 0 || H_kv <= 0 || Nq <= 0 || Nk <= 0 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (mask == FA_MASK_CAUSAL_BOTTOM_RIGHT && Nk < Nq) return FA_ERR_SHAPE;
  if (!head_fits(Nq, d, FA_DTYPE_BF16) || Nk > kI32Max / d) return FA_ERR_SHAPE;  // o in bf16, k/v one byte
  if (B > kI32Max / H || B * H > kI32Max / ((Nq + 31) / 32)) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_ARG;
  int dev = 0, num_cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || num_cus <= 0)
    return FA_ERR_HIP;
  const bool causal = mask != FA_MASK_NONE;
  const int diag = mask == FA_MASK_CAUSAL_BOTTOM_RIGHT ? (int)(Nk - Nq) : 0;
  fa::FwdFp8Args a{q, k, v, q_scale, k_scale, v_scale, o, lse, (int)B, (int)H, (int)Nq, (int)Nk, (int)d, (int)H_kv,
                   causal, diag, scale, num_cus};
  return from_hip(fa::launch_fwd_fp8(a, stream));
}

size_t fa_fwd_masked_workspace_bytes(int64_t Nq, int64_t Nk) {
  if (Nq <= 0 || Nk <= 0 || Nk > (int64_t)fa::kMaxMaskTiles * 64 || Nq > kI32Max) return 0;
  const int64_t n_qblk = (Nq + fa::kFwdBlockRows - 1) / fa::kFwdBlockRows, nT = (Nk + 63) / 64;
  return (size_t)(mask_ws_counts_bytes(n_qblk) + mask_ws_cls_bytes(n_qblk, nT) + mask_ws_lists_bytes(n_qblk, nT) + 16);
}

fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                          int64_t H_kv, int64_t Nq, int64_t Nk, int64_t d, const uint64_t* mask, void* workspace,
                          size_t workspace_bytes, float scale, fa_dtype_t dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !mask || !workspace) return FA_ERR_NULL;
  if (dtype != FA_DTYPE_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(mask, 8) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  if (B <= 0 || H <= 0 || H_kv <= 0 || Nq <= 0 || Nk <= 0 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (Nk > (int64_t)fa::kMaxMaskTiles * 64) return FA_ERR_SHAPE;  // the block's tile list lives in LDS
  if (!head_fits(Nq, d, dtype) || !head_fits(Nk, d, dtype)) return FA_ERR_SHAPE;
  if (B > kI32Max / H || B * H > kI32Max / ((Nq + 31) / 32)) return FA_ERR_SHAPE;
  const int64_t nT = (Nk + 63) / 64;
  if (Nq > kI32Max / nT) return FA_ERR_SHAPE;  // mask word offsets
  if (!scale_ok(scale)) return FA_ERR_ARG;
  if (workspace_bytes < fa_fwd_masked_workspace_bytes(Nq, Nk)) return FA_ERR_WORKSPACE;
  int dev = 0, num_cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || num_cus <= 0)
    return FA_ERR_HIP;
  const int n_qblk = (int)((Nq + fa::kFwdBlockRows - 1) / fa::kFwdBlockRows);
  char* wsb = static_cast<char*>(workspace);
  int* counts = reinterpret_cast<int*>(wsb);
  uint8_t* cls = reinterpret_cast<uint8_t*>(wsb + mask_ws_counts_bytes(n_qblk));
  uint16_t* lists = reinterpret_cast<uint16_t*>(wsb + mask_ws_counts_bytes(n_qblk) + mask_ws_cls_bytes(n_qblk, nT));
  int* queue = reinterpret_cast<int*>(reinterpret_cast<char*>(lists) + mask_ws_lists_bytes(n_qblk, nT));
  fa::MaskClassifyArgs ca{mask, (int)Nq, (int)Nk, (int)nT, fa::kFwdBlockRows, n_qblk, cls, counts, lists, queue};
  fa_status_t st = from_hip(fa::launch_mask_classify(ca, stream));
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, (int)B, (int)H, (int)Nq, (int)Nk, (int)d, (int)H_kv, false, 0, scale, num_cus,
                counts, lists, mask, (int)nT, queue};
  return from_hip(fa::launch_fwd_bf16_masked(a, stream));
}

size_t fa_decode_workspace_bytes(int64_t B, int64_t H, int64_t d, int num_splits) {
  if (B <= 0 || H <= 0 || d <= 0 || num_splits <= 0) return 0;
  if (B > kI32Max / H || B * H > kI32Max / num_splits) return 0;
  return (size_t)(B * H * num_splits) * (size_t)(d + 2) * sizeof(float);
}

fa_status_t fa_decode_split(const void* q, const void* k, const void* v, void* workspace, size_t workspace_bytes,
                            int64_t B, int64_t H, int64_t Nk, int64_t d, float scale, int num_splits,
                            fa_dtype_t dtype, hipStream_t stream) {
  return decode_split(q, k, v, workspace, workspace_bytes, B, H, H, Nk, d, scale, num_splits, dtype, stream);
}

fa_status_t fa_decode_split_ex(const void* q, const void* k, const void* v, void* workspace, size_t workspace_bytes,
                               int64_t B, int64_t H, int64_t H_kv, int64_t Nk, int64_t d, float scale, int num_splits,
                               fa_dtype_t dtype, hipStream_t stream) {
  return decode_split(q, k, v, workspace, workspace_bytes, B, H, H_kv, Nk, d, scale, num_splits, dtype, stream);
}

fa_status_t fa_decode_combine(const void* workspace, size_t workspace_bytes, void* o, float* lse, int64_t B,
                              int64_t H, int64_t d, int num_splits, fa_dtype_t dtype, hipStream_t stream) {
  if (!workspace || !o || !lse) return FA_ERR_NULL;
  if (!dtype_ok(dtype) || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if (!aligned(workspace, 16) || !aligned(o, 16) || !aligned(lse, 4)) return FA_ERR_ALIGN;
  if (B <= 0 || H <= 0 || B > kI32Max / H) return FA_ERR_SHAPE;
  if (num_splits < 1) return FA_ERR_ARG;
  if (B * H > kI32Max / num_splits) return FA_ERR_SHAPE;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const float* o_part = static_cast<const float*>(workspace);
  const float* ml = o_part + (size_t)(B * H * num_splits) * (size_t)d;
  fa::DecodeCombineArgs a{o_part, ml, o, lse, (int)B, (int)H, (int)d, num_splits};
  return from_hip(dtype == FA_DTYPE_BF16 ? fa::launch_decode_combine_bf16(a, stream)
                                         : fa::launch_decode_combine_f32(a, stream));
}

fa_status_t fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                              int64_t H, int64_t H_kv, int64_t Nk, int64_t d, float scale, int num_splits,
                              fa_dtype_t dtype, hipStream_t stream) {
  // Everything is validated before the first HIP call, the scratch address lookup included.
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!dtype_ok(dtype) || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  if (B <= 0 || H <= 0 || H_kv <= 0 || Nk <= 0 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (!head_fits(Nk, d, dtype) || B > kI32Max / H) return FA_ERR_SHAPE;
  if (num_splits < 1 || num_splits > Nk || !scale_ok(scale)) return FA_ERR_ARG;
  if (B * H > kI32Max / num_splits) return FA_ERR_SHAPE;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (need > FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (fa::decode_scratch_address(&ws) != hipSuccess) return FA_ERR_HIP;
  float* o_part = static_cast<float*>(ws);
  float* ml = o_part + (size_t)(B * H * num_splits) * (size_t)d;
  const bool bf16 = dtype == FA_DTYPE_BF16;
  fa::DecodeSplitArgs sa{q, k, v, o_part, ml, (int)B, (int)H, (int)Nk, (int)d, num_splits, (int)H_kv, scale};
  const fa_status_t st = from_hip(bf16 ? fa::launch_decode_split_bf16(sa, stream)
                                       : fa::launch_decode_split_f32(sa, stream));
  if (st != FA_OK) return st;
  fa::DecodeCombineArgs ca{o_part, ml, o, lse, (int)B, (int)H, (int)d, num_splits};
  return from_hip(bf16 ? fa::launch_decode_combine_bf16(ca, stream) : fa::launch_decode_combine_f32(ca, stream));
}

fa_status_t fa_decode_split_fp8kv(const void* q, const void* k, const void* v, const float* k_scale,
                                  const float* v_scale, void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                                  int64_t H_kv, int64_t Nk, int64_t d, float scale, int num_splits,
                                  hipStream_t stream) {
  if (!q || !k || !v || !k_scale || !v_scale || !workspace) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(workspace, 16) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4))
    return FA_ERR_ALIGN;
  if (B <= 0 || H <= 0 || H_kv <= 0 || Nk <= 0 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (Nk > kI32Max / d || B > kI32Max / H) return FA_ERR_SHAPE;  // one head of codes: 32-bit offsets
  if (num_splits < 1 || num_splits > Nk || !scale_ok(scale)) return FA_ERR_ARG;
  if (B * H > kI32Max / num_splits) return FA_ERR_SHAPE;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  float* o_part = static_cast<float*>(workspace);
  float* ml = o_part + (size_t)(B * H * num_splits) * (size_t)d;
  fa::DecodeSplitFp8Args a{q, k, v, k_scale, v_scale, o_part, ml, (int)B, (int)H, (int)Nk, (int)d, num_splits,
                           (int)H_kv, scale};
  return from_hip(fa::launch_decode_split_fp8kv(a, stream));
}

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq) {
  if (B <= 0 || H <= 0 || Nq <= 0 || B > kI32Max / H || B * H > kI32Max / Nq) return 0;
  return (size_t)(B * H * Nq) * 2 * sizeof(float);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                   int64_t H_kv, int64_t Nq, int64_t Nk, int64_t d, fa_mask_t mask, float scale, fa_dtype_t dtype,
                   hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  if (dtype != FA_DTYPE_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_CAUSAL_BOTTOM_RIGHT) return FA_ERR_ARG;
  if (B <= 0 || H <= 0 || H_kv <= 0 || Nq <= 0 || Nk <= 0 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (mask == FA_MASK_CAUSAL_BOTTOM_RIGHT && Nk < Nq) return FA_ERR_SHAPE;
  if (!head_fits(Nq, d, dtype) || !head_fits(Nk, d, dtype)) return FA_ERR_SHAPE;
  // the workspace (2 floats per query row) is addressed with 32-bit byte offsets
  if (B > kI32Max / H || B * H > kI32Max / 8 / Nq) return FA_ERR_SHAPE;
  if (!scale_ok(scale)) return FA_ERR_ARG;
  if (workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq)) return FA_ERR_WORKSPACE;
  const bool causal = mask != FA_MASK_NONE;
  const int diag = mask == FA_MASK_CAUSAL_BOTTOM_RIGHT ? (int)(Nk - Nq) : 0;
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace), (int)B, (int)H, (int)Nq, (int)Nk,
                (int)d, (int)H_kv, causal, diag, scale};
  return from_hip(fa::launch_bwd_bf16(a, stream));
}

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_ALIGN: return "pointer misaligned (tensors need 16 bytes, lse 4 bytes)";
    case FA_ERR_SHAPE:
      return "invalid shape (size <= 0, H_kv not dividing H, a causal alignment some row sees no key under, "
             "or beyond index limits)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim (64 or 128) or dtype";
    case FA_ERR_WORKSPACE: return "workspace smaller than the size its *_workspace_bytes function returns";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    case FA_ERR_ARG:
      return "invalid scalar argument (scale must be finite and > 0; 1 <= num_splits <= Nk; known mask)";
    case FA_ERR_SCRATCH:
      return "decode partials larger than the fixed scratch of fa_decode_noalloc (FA_DECODE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"
