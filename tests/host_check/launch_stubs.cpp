// Launch stubs for a host-only build of the C-ABI layer (fa_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU.  Each stub answers as a launch does in a process without
// a GPU: hipErrorNoDevice, which the layer reports as FA_ERR_HIP.  The validation cases expect
// their own status codes, so an argument that should be rejected but reached a launch fails its
// case.  Test infrastructure only; the library's real launchers live in the .hip files.
#include "fa_launch.h"

namespace fa {
hipError_t launch_fwd_bf16(const FwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fwd_f32(const FwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_split_bf16(const DecodeSplitArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_split_f32(const DecodeSplitArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_combine_bf16(const DecodeCombineArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_combine_f32(const DecodeCombineArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_bf16(const BwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_split_fp8kv(const DecodeSplitFp8Args&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fwd_fp8(const FwdFp8Args&, hipStream_t) { return hipErrorNoDevice; }
hipError_t decode_scratch_address(void**) { return hipErrorNoDevice; }
hipError_t launch_mask_classify(const MaskClassifyArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fwd_bf16_masked(const FwdArgs&, hipStream_t) { return hipErrorNoDevice; }
}  // namespace fa
