// Tile classification for the masked forward (fa_fwd_masked).
//
// The forward skips key tiles that a mask leaves empty for a whole query block and masks element
// by element only the tiles that are partly visible (Day-21 page "GPU 学习日报 Day 21：
// FlashAttention：GPU Memory Hierarchy 下的 IO 优化", §6 table, last row).  These two kernels read
// the bit-packed element mask once and leave, per query block of `br` rows, the key-ordered list of
// its non-empty 64-key tiles (bit 15 set on a partial one) and their count; the forward walks that
// list instead of a range of tiles.
//
// mask_classify_kernel: one workgroup of four waves per (query block, 64 consecutive tiles).  Lane
// l of every wave takes tile 64 * blockIdx.y + l; wave w ANDs and ORs the mask words of rows w,
// w + 4, ... of the block (consecutive lanes read consecutive words of a row: 512 contiguous bytes
// per wave and row), restricted to the keys below Nk and the rows below Nq; the four waves combine
// through LDS and the first writes one class byte per tile: 0 empty, 1 full, 2 partial.
// mask_compact_kernel: one wave per query block compacts the class bytes into the list, in key
// order, with a ballot per 64 tiles.
// The classification also zeroes the counter from which the forward's workgroups claim their
// (query block, head) items.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

__global__ __launch_bounds__(256) void mask_classify_kernel(const uint64_t* __restrict__ mask, int Nq, int Nk,
                                                            int nT, int br, uint8_t* __restrict__ cls,
                                                            int* __restrict__ queue) {
  const int qb = blockIdx.x;
  if (qb == 0 && blockIdx.y == 0 && threadIdx.x == 0) *queue = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.y * 64 + lane;
  const int r0 = qb * br, r1 = min(Nq, r0 + br);
  uint64_t all = ~0ull, any = 0;
  if (t < nT) {
    const int keys = min(64, Nk - 64 * t);
    const uint64_t valid = keys == 64 ? ~0ull : ((1ull << keys) - 1ull);
    all = valid;
    const uint64_t* p = mask + (int64_t)(r0 + wave) * nT + t;
#pragma unroll 8
    for (int r = r0 + wave; r < r1; r += 4, p += 4 * (int64_t)nT) {
      const uint64_t w = *p & valid;
      all &= w;
      any |= w;
    }
    all ^= valid;  // the valid keys some row does not see
  }
  __shared__ uint64_t part[2][4][64];
  part[0][wave][lane] = all;
  part[1][wave][lane] = any;
  __syncthreads();
  if (wave == 0 && t < nT) {
    const uint64_t missing = part[0][0][lane] | part[0][1][lane] | part[0][2][lane] | part[0][3][lane];
    const uint64_t seen = part[1][0][lane] | part[1][1][lane] | part[1][2][lane] | part[1][3][lane];
    cls[(int64_t)qb * nT + t] = seen == 0 ? 0 : (missing == 0 ? 1 : 2);
  }
}

__global__ __launch_bounds__(64) void mask_compact_kernel(const uint8_t* __restrict__ cls, int nT,
                                                          int* __restrict__ counts, uint16_t* __restrict__ lists) {
  const int qb = blockIdx.x, lane = threadIdx.x;
  const uint8_t* c = cls + (int64_t)qb * nT;
  uint16_t* lst = lists + (int64_t)qb * nT;
  int base = 0;
  for (int t0 = 0; t0 < nT; t0 += 64) {
    const int t = t0 + lane;
    const int k = t < nT ? c[t] : 0;
    const uint64_t b = __ballot(k != 0);
    if (k != 0) lst[base + __popcll(b & ((1ull << lane) - 1ull))] = (uint16_t)(t | (k == 2 ? 0x8000 : 0));
    base += __popcll(b);
  }
  if (lane == 0) counts[qb] = base;
}

}  // namespace

hipError_t launch_mask_classify(const MaskClassifyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mask_classify_kernel, dim3((unsigned)a.n_qblk, (unsigned)((a.nT + 63) / 64)), dim3(256), 0,
                     stream, a.mask, a.Nq, a.Nk, a.nT, a.br, a.cls, a.queue);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mask_compact_kernel, dim3((unsigned)a.n_qblk), dim3(64), 0, stream, a.cls, a.nT, a.counts,
                     a.lists);
  return hipGetLastError();
}

}  // namespace fa
