// Internal interface between the C-ABI layer (fa_api.cpp) and the kernel files.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Size of the fixed device scratch behind fa_decode_noalloc (its split partials).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
// Query rows per block of the bf16 forward, the granularity of the mask classification.
constexpr int kFwdBlockRows = 256;
// Largest number of 64-key tiles per row the masked forward takes (its block's tile list is held
// in LDS): Nk <= 131072.
constexpr int kMaxMaskTiles = 2048;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk, d;
  int H_kv;    // K/V heads; divides H, query head h reads K/V head h / (H / H_kv)
  bool causal;
  int diag;    // causal: key j visible to query i iff j <= i + diag (0 top-left, Nk - Nq bottom-right)
  float scale;
  int num_cus;  // compute units of the device the stream runs on (persistent grid size)
  // masked forward only (null / 0 otherwise): per query block of kFwdBlockRows rows the number and
  // list of non-empty 64-key tiles (bit 15 = partial), and the bit-packed element mask
  const int* mask_counts = nullptr;
  const uint16_t* mask_lists = nullptr;
  const uint64_t* mask_words = nullptr;
  int mask_tiles = 0;  // 64-key tiles per row, ceil(Nk / 64)
  // the counter from which the workgroups claim (query block, head) items
  int* mask_queue = nullptr;
};

struct MaskClassifyArgs {
  const uint64_t* mask;  // [Nq][nT] bit-packed element mask
  int Nq, Nk, nT, br, n_qblk;
  uint8_t* cls;     // [n_qblk][nT] class of each tile: 0 empty, 1 full, 2 partial
  int* counts;      // [n_qblk]
  uint16_t* lists;  // [n_qblk][nT]
  int* queue;       // the forward's claim counter (dynamic item schedule), zeroed by the classification
};

struct FwdFp8Args {
  const void* q;  // E4M3 codes [B][H][Nq][d]
  const void* k;  // E4M3 codes [B][H_kv][Nk][d]
  const void* v;
  const float* q_scale;  // [B][H]
  const float* k_scale;  // [B][H_kv]
  const float* v_scale;
  void* o;  // bf16 [B][H][Nq][d]
  float* lse;
  int B, H, Nq, Nk, d;
  int H_kv;
  bool causal;
  int diag;
  float scale;
  int num_cus;
};

struct DecodeSplitArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o_part;  // [B][H][S][d]
  float* ml;      // [B][H][S][2]
  int B, H, Nk, d, num_splits;
  int H_kv;       // K/V heads; divides H, query head h reads K/V head h / (H / H_kv)
  float scale;
};

struct DecodeSplitFp8Args {
  const void* q;        // bf16 [B][H][1][d]
  const void* k;        // E4M3 codes [B][H_kv][Nk][d]
  const void* v;
  const float* k_scale;  // [B][H_kv]
  const float* v_scale;
  float* o_part;
  float* ml;
  int B, H, Nk, d, num_splits;
  int H_kv;
  float scale;
};

struct DecodeCombineArgs {
  const float* o_part;
  const float* ml;
  void* o;
  float* lse;
  int B, H, d, num_splits;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // forward's per-row LSE, natural-log units
  void* dq;
  void* dk;
  void* dv;
  float* ws;  // [2][B][H][Nq]: LSE in log2 units, then rowsum(dO * O)
  int B, H, Nq, Nk, d;
  int H_kv;
  bool causal;
  int diag;
  float scale;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_mask_classify(const MaskClassifyArgs& a, hipStream_t stream);
hipError_t launch_fwd_bf16_masked(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode_split_bf16(const DecodeSplitArgs& a, hipStream_t stream);
hipError_t launch_decode_split_f32(const DecodeSplitArgs& a, hipStream_t stream);
hipError_t launch_decode_combine_bf16(const DecodeCombineArgs& a, hipStream_t stream);
hipError_t launch_decode_combine_f32(const DecodeCombineArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_decode_split_fp8kv(const DecodeSplitFp8Args& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const FwdFp8Args& a, hipStream_t stream);
// Device address of the fixed decode scratch on the current device (looked up on first use).
hipError_t decode_scratch_address(void** out);

}  // namespace fa
