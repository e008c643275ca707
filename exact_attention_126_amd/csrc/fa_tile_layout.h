// LDS tile layout and MFMA row order shared by the forward and backward kernels.
#pragma once

namespace fa {

// XOR swizzle applied to the 16-byte chunk index of an LDS row of D bf16 values, from the row's
// low 4 bits.  Chosen so that the 32x32x16 MFMA operand reads of a 64-row tile (16-byte row
// reads of 32 rows at one chunk, and the transposing 8-byte reads) and the 1 KiB LDS DMA stores
// are free of bank conflicts.
template <int D> struct Swz;
template <> struct Swz<128> { static constexpr int b0 = 4, b1 = 10, b2 = 1, b3 = 3; };
template <> struct Swz<64> { static constexpr int b0 = 2, b1 = 4, b2 = 1, b3 = 3; };

template <int D>
__device__ __forceinline__ int swz(int row) {
  return ((row & 1) ? Swz<D>::b0 : 0) ^ ((row & 2) ? Swz<D>::b1 : 0) ^
         ((row & 4) ? Swz<D>::b2 : 0) ^ ((row & 8) ? Swz<D>::b3 : 0);
}

// The 32x32 MFMA accumulator holds row r = 8*(j/4) + 4*h + (j%4) in register j of lane-half h.
// key_of_row(r) is the key loaded for row r so that register j of lane-half h is key
// 16*(j/8) + 8*h + (j%8) of the 32-key block: then 8 consecutive accumulator registers, packed
// to bf16, are the B operand of the next MFMA whose k index runs over those keys.
__device__ __forceinline__ int key_of_row(int r) {
  const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

}  // namespace fa
