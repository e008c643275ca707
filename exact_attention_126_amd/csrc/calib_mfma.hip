// Sustained dense bf16 matrix-core rate of the GPU under its own power management.  Every SIMD
// runs one wave that issues v_mfma_f32_32x32x16_bf16 back to back (four independent
// accumulators) on operands taken from the caller's buffer, so the operand bit patterns
// (and with them the energy per instruction) are whatever the caller supplies.  The nominal
// peak assumes the 2.4 GHz maximum engine clock; under a long run of matrix instructions the
// clock settles lower, and this kernel measures where.  A measurement aid for the forward
// kernel's roofline, built into its own library; the attention path does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Four waves per workgroup and one workgroup per CU (the caller's grid): one wave per SIMD.  Two
// waves streaming MFMAs on one SIMD contend for its matrix core and are arbitrated unevenly.
constexpr int kThreads = 256;
constexpr int kFragsPerWg = 8;  // four A and four B fragments, 64 lanes x 16 bytes each

// clk[2b] = shader-clock cycles (s_memtime) and clk[2b + 1] = 100 MHz reference ticks
// (s_memrealtime) spent by workgroup b in its MFMA loop.
__global__ __launch_bounds__(kThreads) void mfma_ceiling_kernel(const u32x4_t* __restrict__ src,
                                                              float* __restrict__ out,
                                                              unsigned long long* __restrict__ clk, int niter) {
  const int lane = threadIdx.x & 63;
  const u32x4_t* s = src + (size_t)blockIdx.x * kFragsPerWg * 64;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8_t, s[i * 64 + lane]);
    b[i] = __builtin_bit_cast(bf16x8_t, s[(4 + i) * 64 + lane]);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
  __syncthreads();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), w0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < niter; it += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + r) & 3], acc[i], 0, 0, 0);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), w1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += acc[i][j];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = sum;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = c1 - c0;
    clk[2 * blockIdx.x + 1] = w1 - w0;
  }
}

}  // namespace

extern "C" {

// Bytes of operand buffer, and floats of output buffer, that fa_calib_mfma needs for `grid`
// workgroups.
size_t fa_calib_src_bytes(int grid) { return grid > 0 ? (size_t)grid * kFragsPerWg * 64 * 16 : 0; }
size_t fa_calib_out_floats(int grid) { return grid > 0 ? (size_t)grid * kThreads : 0; }

// Launches `grid` workgroups of the loop above; each of a workgroup's four waves issues
// 4 * niter MFMAs (niter a positive multiple of 4).  src: device buffer of at least fa_calib_src_bytes(grid) bytes (16-byte
// aligned); out: device buffer of fa_calib_out_floats(grid) floats; clk: device buffer of 2 * grid
// unsigned 64-bit counters.  Returns 0, or -1 for bad arguments (nothing launched), or the HIP
// error code of the launch.
int fa_calib_mfma(const void* src, size_t src_bytes, float* out, size_t out_floats, unsigned long long* clk,
                  int grid, int niter, hipStream_t stream) {
  if (!src || !out || !clk || grid <= 0 || niter <= 0 || niter % 4 != 0) return -1;
  if (((uintptr_t)src & 15) != 0 || src_bytes < fa_calib_src_bytes(grid) || out_floats < fa_calib_out_floats(grid))
    return -1;
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(grid), dim3(kThreads), 0, stream, (const u32x4_t*)src, out, clk, niter);
  return (int)hipGetLastError();
}

}  // extern "C"
