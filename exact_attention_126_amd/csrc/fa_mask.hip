// Tile classification for the masked forward (fa_fwd_masked).
//
// The forward skips key tiles that a mask leaves empty for a whole query block and masks element
// by element only the tiles that are partly visible (Day-21 page "GPU 学习日报 Day 21：
// FlashAttention：GPU Memory Hierarchy 下的 IO 优化", §6 table, last row).  This pass reads the
// bit-packed element mask once and, for every query block of BR rows and every 64-key tile,
// decides which of the three the tile is, then writes per block the list of its non-empty tiles
// in key order, each with a flag for "partial", and their count.  The forward then walks that
// list instead of a range.
//
// mask_classify_kernel: one workgroup of 256 threads per query block.  Thread t takes tiles
// t, t + 256, ...; for its tile it ANDs and ORs the block's mask words (consecutive threads read
// consecutive words of a row, so a wave reads 512 contiguous bytes per row), restricted to the
// keys below Nk and the rows below Nq.  The non-empty tiles are compacted in key order with a wave
// ballot and a prefix over the four waves.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

__global__ __launch_bounds__(256) void mask_classify_kernel(const uint64_t* __restrict__ mask, int Nq, int Nk,
                                                            int nT, int br, int* __restrict__ counts,
                                                            uint16_t* __restrict__ lists) {
  const int qb = blockIdx.x;
  const int r0 = qb * br, r1 = min(Nq, r0 + br);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int wsum[4];
  int base = 0;
  for (int t0 = 0; t0 < nT; t0 += 256) {
    const int t = t0 + tid;
    int cls = 0;  // 0 empty, 1 full, 2 partial
    if (t < nT) {
      const int keys = min(64, Nk - 64 * t);
      const uint64_t valid = keys == 64 ? ~0ull : ((1ull << keys) - 1ull);
      uint64_t all = valid, any = 0;
      const uint64_t* p = mask + (int64_t)r0 * nT + t;
      for (int r = r0; r < r1; ++r, p += nT) {
        const uint64_t w = *p & valid;
        all &= w;
        any |= w;
      }
      cls = any == 0 ? 0 : (all == valid ? 1 : 2);
    }
    const uint64_t b = __ballot(cls != 0);
    const int before = __popcll(b & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(b);
    __syncthreads();
    int off = base;
    for (int i = 0; i < wave; ++i) off += wsum[i];
    if (cls != 0) lists[(int64_t)qb * nT + off + before] = (uint16_t)(t | (cls == 2 ? 0x8000 : 0));
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (tid == 0) counts[qb] = base;
}

}  // namespace

hipError_t launch_mask_classify(const MaskClassifyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mask_classify_kernel, dim3((unsigned)a.n_qblk), dim3(256), 0, stream, a.mask, a.Nq, a.Nk,
                     a.nT, a.br, a.counts, a.lists);
  return hipGetLastError();
}

}  // namespace fa
