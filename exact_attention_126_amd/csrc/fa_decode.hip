// Split-KV decode for gfx950: one query token per (batch, head) against a long KV cache.
//
// Decode is a matrix-vector product bound by reading the KV cache from HBM (Day-21 page
// "GPU 学习日报 Day 21：FlashAttention：GPU Memory Hierarchy 下的 IO 优化", §9 and FAQ Q5), so
// one query head per K/V head runs on the VALU; only grouped heads (several query rows per K/V
// row) use the matrix core.  The work is spread over many workgroups by splitting the keys into
// contiguous chunks that are processed in parallel and merged afterwards (Q31 answer
// "FlashAttention 为什么快", follow-up 3).  The merge rescales every partial result by
// exp(m_s - max m) before summing (same answer, follow-up 2).
//
// decode_split_kernel: one workgroup per (batch, group of query heads sharing a K/V head, split).
// D/8 (bf16) or D/4 (fp32) lanes share a key row and read it with coalesced 16-byte loads; each
// wave walks its own keys with an online softmax per query head (running max, running sum,
// rescaled accumulator, Day-21 page §5.2-5.3), U key rows of K and of V in flight per lane.
// With grouped K/V heads (several query heads per K/V head, which the Day-21 page's FAQ Q5
// names among the decode-side techniques) a workgroup serves up to four query heads from one
// read of the K/V rows (for bf16: decode_split_mfma_kernel).  The four waves' states are merged
// through LDS and written to the workspace as (O_part, m, l) per query head.
// decode_combine_kernel: one workgroup per (batch*head), one thread per dim.
#include <atomic>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

// 16-byte load of K/V cache data that is read exactly once: the non-temporal hint keeps the stream
// from displacing reusable lines (the split partials the combine reads next) in the caches.
__device__ __forceinline__ u32x4_t stream_load16(const void* p) {
  return __builtin_nontemporal_load((const u32x4_t*)p);
}
// The same hint as the cache-policy operand of a buffer load (the NT bit)
constexpr int kNonTemporal = 2;

// x from lane CTRL-permuted within its row.  Every pattern used here reads a valid lane, so
// bound_ctrl is set: that lets the compiler fold the move into the add that consumes it
// (v_add_f32 with a DPP source) instead of issuing a separate v_mov_b32_dpp.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over aligned groups of W consecutive lanes (W in {4, 8, 16, 32}); every lane gets the sum.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  if (W >= 8) x += dpp<kRowHalfMirror>(x);  // pairs quad 0 with quad 1 of each 8 lanes
  if (W >= 16) x += dpp<kRowMirror>(x);  // pairs the two 8-lane halves of each row
  if (W >= 32) x += __shfl_xor(x, 16);
  return x;
}

// max / sum of x over lanes l and l ^ W.  W = 16 and 32 stay in the VALU (v_permlane16_swap /
// v_permlane32_swap hand each lane its partner's value next to its own); smaller W go through
// the LDS crossbar.  Both operands are commutative, so every form gives the same bits.
template <int W>
__device__ __forceinline__ float xor_max(float x) {
  if constexpr (W == 16 || W == 32) {
    const auto r = W == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                           : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    return fmaxf(x, __shfl_xor(x, W));
  }
}
template <int W>
__device__ __forceinline__ float xor_sum(float x) {
  if constexpr (W == 16 || W == 32) {
    const auto r = W == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                           : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return x + __shfl_xor(x, W);
  }
}
// Reduction over the lanes l ^ W, l ^ 2W, ... up to l ^ 32 (the key-row groups of a wave).
template <int W>
__device__ __forceinline__ float max_over_groups(float x) {
  if constexpr (W >= 64) {
    return x;
  } else {
    return max_over_groups<2 * W>(xor_max<W>(x));
  }
}
template <int W>
__device__ __forceinline__ float sum_over_groups(float x) {
  if constexpr (W >= 64) {
    return x;
  } else {
    return sum_over_groups<2 * W>(xor_sum<W>(x));
  }
}

template <typename T>
struct Elt;
template <>
struct Elt<uint16_t> {  // bf16 storage
  static constexpr int PER16 = 8;
  __device__ static void widen(u32x4_t r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
  __device__ static uint16_t narrow(float x) { return f32_to_bf16_bits(x); }
};
template <>
struct Elt<float> {
  static constexpr int PER16 = 4;
  __device__ static void widen(u32x4_t r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
  }
  __device__ static float narrow(float x) { return x; }
};

// One workgroup per (batch, group of GE query heads that share a K/V head, split): the K/V rows
// of the split are read once and serve all GE heads.  Each head's arithmetic is the same
// whatever GE is (per-head dot products, maxima, sums and accumulators in the same order), so a
// grouped call gives bit for bit what an ungrouped call on repeated K/V heads gives.
template <typename T, int D, int GE>
__global__ __launch_bounds__(256) void decode_split_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                           const T* __restrict__ V, float* __restrict__ Opart,
                                                           float* __restrict__ ML, int Nk, int S, int chunk,
                                                           float sl2, int H, int group) {
  constexpr int EPL = Elt<T>::PER16;  // elements per lane per key row
  constexpr int LPK = D / EPL;        // lanes per key row
  constexpr int KPW = 64 / LPK;       // key rows per wave per step
  constexpr int U = 16;               // steps in flight per iteration (the same for every GE)
  constexpr int WAVES = 4;
  __shared__ float s_m[WAVES][GE], s_l[WAVES][GE];
  __shared__ float s_acc[WAVES][GE][D];

  const int s = blockIdx.x % S;
  const int bh0 = (blockIdx.x / S) * GE;  // first query head (b * H + h) of this workgroup's group
  const int start = s * chunk;
  const int end = min(Nk, start + chunk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int gi = lane / LPK, li = lane % LPK;

  float qv[GE][EPL];
#pragma unroll
  for (int g = 0; g < GE; ++g) {
    Elt<T>::widen(gload16(Q + (int64_t)(bh0 + g) * D + li * EPL), qv[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[g][e] *= sl2;  // scores come out in log2 units
  }
  const int kvh = (bh0 / H) * (H / group) + (bh0 % H) / group;  // K/V head shared by the GE query heads
  const T* Kh = K + (int64_t)kvh * Nk * D + li * EPL;
  const T* Vh = V + (int64_t)kvh * Nk * D + li * EPL;

  float m[GE], l[GE], acc[GE][EPL];
#pragma unroll
  for (int g = 0; g < GE; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  for (int base = start + wave * U * KPW; base < end; base += WAVES * U * KPW) {
    u32x4_t kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(base + u * KPW + gi, end - 1);
      kr[u] = stream_load16(Kh + (int64_t)key * D);
      vr[u] = stream_load16(Vh + (int64_t)key * D);
    }
    float sc[U][GE];
    float bm[GE];
#pragma unroll
    for (int g = 0; g < GE; ++g) bm[g] = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      Elt<T>::widen(kr[u], kf);
      const bool in = base + u * KPW + gi < end;
#pragma unroll
      for (int g = 0; g < GE; ++g) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[g][e], kf[e], dot);
        dot = group_sum<LPK>(dot);
        sc[u][g] = in ? dot : -INFINITY;
        bm[g] = fmaxf(bm[g], sc[u][g]);
      }
    }
#pragma unroll
    for (int g = 0; g < GE; ++g) {
      bm[g] = max_over_groups<LPK>(bm[g]);
      const float mnew = fmaxf(m[g], bm[g]);
      const float alpha = fast_exp2(m[g] - mnew);
      m[g] = mnew;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      Elt<T>::widen(vr[u], vf);
#pragma unroll
      for (int g = 0; g < GE; ++g) {
        const float p = fast_exp2(sc[u][g] - m[g]);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = __builtin_fmaf(p, vf[e], acc[g][e]);
      }
    }
  }
  // fold the key groups of the wave: lanes with equal li hold the same dims
#pragma unroll
  for (int g = 0; g < GE; ++g) {
    l[g] = sum_over_groups<LPK>(l[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = sum_over_groups<LPK>(acc[g][e]);
    if (lane == 0) {
      s_m[wave][g] = m[g];
      s_l[wave][g] = l[g];
    }
    if (gi == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][g][li * EPL + e] = acc[g][e];
    }
  }
  __syncthreads();
  for (int x = tid; x < GE * D; x += 256) {
    const int g = x / D, dim = x % D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) M = fmaxf(M, s_m[w][g]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = fast_exp2(s_m[w][g] - M);
        o = __builtin_fmaf(f, s_acc[w][g][dim], o);
        L = __builtin_fmaf(f, s_l[w][g], L);
      }
    }
    const int64_t rec = (int64_t)(bh0 + g) * S + s;
    Opart[rec * D + dim] = o;
    if (dim == 0) {
      ML[rec * 2] = (M == -INFINITY) ? -INFINITY : M * kLn2;
      ML[rec * 2 + 1] = L;
    }
  }
}

// Grouped decode on the matrix core (bf16 K/V, GE = 2 or 4 query heads per K/V head).  With
// several query heads per K/V row, the kernel above spends most of its time on per-head dot
// products and accumulations on the VALU; here both products run on v_mfma_f32_16x16x32_bf16,
// with the GE query rows padded to 16:
//  * S^T = K Q^T, one 16-key tile by 16 query columns per MFMA.  Lane l takes key row l % 16 of
//    the tile and dims 32 ks + 8 (l / 16) .. + 7 of it as its A operand straight from HBM (each
//    row group of four lanes reads 64 contiguous bytes per k-step), and the same dims of query
//    l % 16 as B.  The accumulator gives lane l query l % 16 against keys 4 (l / 16) .. + 3.
//  * One exact row max per 32-key trip (in the lane, then over the four lane groups), and P =
//    exp2(S scale log2 e - m) packed to bf16 straight from the accumulators: the keys
//    16 (e / 4) + 4 (l / 16) + e % 4 of the trip (e = 0..7) that lane l holds are its B operand of
//  * O^T += V^T P^T, 16 dims by 16 query columns per MFMA.  V goes by LDS DMA into a buffer of
//    the wave's own, and its A operand (dim 16 mb + l % 16 of those same eight keys) comes from
//    two transposing ds_read_b64_tr_b16 reads.  O^T's lane l holds query l % 16, so the rescale by
//    exp2(m_old - m_new) is a per-lane scalar.
// Rows of the V buffers are XOR-swizzled in 16-byte chunks by the row's low bits.  Each wave loads
// one trip at a time (its K rows into registers, its V rows into its buffer) and computes it; three
// workgroups per compute unit keep other waves' loads in flight meanwhile.  The four waves merge
// their states through LDS as in the kernel above and write the same partials.
#ifndef FA_DEC_TRIP
#define FA_DEC_TRIP 32  // keys per wave per trip of the matrix-core decode split
#endif

template <int D, int GE>
__global__ __launch_bounds__(256) void decode_split_mfma_kernel(const uint16_t* __restrict__ Q,
                                                                const uint16_t* __restrict__ K,
                                                                const uint16_t* __restrict__ V,
                                                                float* __restrict__ Opart, float* __restrict__ ML,
                                                                int Nk, int S, int chunk, float sl2, int H, int group) {
  constexpr int WAVES = 4, TK = FA_DEC_TRIP;  // keys per wave per trip
  constexpr int NT = TK / 16, NKK = TK / 32;  // 16-key tiles of S^T, 32-key k-steps of O^T per trip
  constexpr int RB = D * 2, CPR = D / 8;      // bytes and 16-byte chunks per key row
  constexpr int KS = D / 32;                  // k-steps of S^T
  constexpr int DB = D / 16;                  // 16-dim blocks of O^T
  constexpr int VDMA = TK * RB / 1024;        // 1 KiB LDS loads per V tile
  static_assert(GE == 2 || GE == 4, "two or four query heads per workgroup");
  static_assert(TK % 32 == 0, "whole k-steps of O^T");
  __shared__ __attribute__((aligned(1024))) char vbuf[WAVES][TK * RB];
  __shared__ float s_m[WAVES][GE], s_l[WAVES][GE];
  __shared__ float s_acc[WAVES][GE][D];

  const int s = blockIdx.x % S;
  const int bh0 = (blockIdx.x / S) * GE;  // first query head (b * H + h) of this workgroup's group
  const int start = s * chunk;
  const int end = min(Nk, start + chunk);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the V loads' resource and LDS base
  const int c16 = lane & 15, G = lane >> 4;
  const int kvh = (bh0 / H) * (H / group) + (bh0 % H) / group;  // K/V head shared by the GE query heads
  const uint16_t* Kh = K + (int64_t)kvh * Nk * D;
  const uint16_t* Vh = V + (int64_t)kvh * Nk * D;

  // Q^T (B operand of S^T): query c16 (zero columns past GE), dims 32 ks + 8 G .. + 7
  u32x4_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
  if (c16 < GE) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = gload16(Q + (int64_t)(bh0 + c16) * D + 32 * ks + 8 * G);
  }
  // transposing V reads: lane (G, c16) of read (mb, I) addresses row 16 I + 4 G + c16 / 4 of a
  // 32-key k-step, dims 16 mb + 4 (c16 % 4) .. + 3, and receives dim 16 mb + c16 of its four rows
  int voff[DB][2];
#pragma unroll
  for (int mb = 0; mb < DB; ++mb)
#pragma unroll
    for (int I = 0; I < 2; ++I) {
      const int row = 16 * I + 4 * G + (c16 >> 2);
      const int byte = (16 * mb + 4 * (c16 & 3)) * 2;
      voff[mb][I] = row * RB + (((byte >> 4) ^ (row % CPR)) << 4) + (byte & 15);
    }

  f32x4_t oT[DB];  // O^T: query c16, dims 16 mb + 4 G + j
#pragma unroll
  for (int mb = 0; mb < DB; ++mb) oT[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running max (log2 units) of query c16, this lane's share of its sum
  const FA_LDS char* vb = (const FA_LDS char*)vbuf[wave];

  for (int base = start + wave * TK; base < end; base += WAVES * TK) {
    // K rows into the A operands of S^T (tile t, k-step ks: key row base + 16 t + c16, dims
    // 32 ks + 8 G), then the V rows into the wave's buffer by LDS DMA (instruction i moves 1 KiB,
    // lane L landing in row (1024 i + 16 L) / RB, slot L % CPR, which holds the row's chunk
    // (L % CPR) ^ (row % CPR); rows past the last key read as zero)
    u32x4_t kr[NT][KS];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint16_t* kp = Kh + (int64_t)min(base + 16 * t + c16, Nk - 1) * D + 8 * G;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[t][ks] = stream_load16(kp + 32 * ks);
    }
    {
      const __amdgpu_buffer_rsrc_t vr = raw_rsrc(Vh + (int64_t)base * D, (Nk - base) * RB);
#pragma unroll
      for (int i = 0; i < VDMA; ++i) {
        const int row = (i * 1024 + lane * 16) / RB;
        const int off = row * RB + (((lane % CPR) ^ (row % CPR)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lptr_t)(vbuf[wave] + i * 1024), 16, off, 0, 0, kNonTemporal);
      }
    }
    f32x4_t st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[t][ks]), as_bf16x8(qf[ks]), st[t], 0, 0, 0);
    }
    if (base + TK > end) {  // keys past the split's end
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (base + 16 * t + 4 * G + j >= end) st[t][j] = -INFINITY;
    }
    // the trip's max of query c16: in the lane, then over the four lane groups
    float mx = st[0][0];
#pragma unroll
    for (int x = 1; x + 1 < 4 * NT; x += 2) mx = max3f(mx, st[x / 4][x % 4], st[(x + 1) / 4][(x + 1) % 4]);
    mx = fmaxf(mx, st[NT - 1][3]);
    mx = xor_max<32>(xor_max<16>(mx));
    const float mnew = fmaxf(m, mx * sl2);
    const float nm = -mnew;  // the trip holds at least one visible key, so mnew is finite
    const float alpha = fast_exp2(m + nm);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int mb = 0; mb < DB; ++mb) oT[mb] *= alpha;
    float p[NT][4];
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[t][j] = fast_exp2(__builtin_fmaf(st[t][j], sl2, nm));
        ps += p[t][j];
      }
    l += ps;
    // B operand of k-step kk (k = keys 32 kk + 16 (e / 4) + 4 G + e % 4 of the trip, e = 0..7)
    u32x4_t pb[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      pb[kk][0] = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
      pb[kk][1] = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
      pb[kk][2] = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
      pb[kk][3] = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the V rows have landed in this wave's buffer
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int mb = 0; mb < DB; ++mb) {
        const i16x4_t lo = lds_load8_tr16(vb + kk * 32 * RB + voff[mb][0]);
        const i16x4_t hi = lds_load8_tr16(vb + kk * 32 * RB + voff[mb][1]);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oT[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(pb[kk]), oT[mb], 0, 0, 0);
      }
  }
  l = xor_sum<32>(xor_sum<16>(l));
  if (lane < GE) {
    s_m[wave][lane] = m;
    s_l[wave][lane] = l;
  }
  if (c16 < GE) {
#pragma unroll
    for (int mb = 0; mb < DB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_acc[wave][c16][16 * mb + 4 * G + j] = oT[mb][j];
  }
  __syncthreads();
  for (int x = tid; x < GE * D; x += 256) {
    const int g = x / D, dim = x % D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) M = fmaxf(M, s_m[w][g]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = fast_exp2(s_m[w][g] - M);
        o = __builtin_fmaf(f, s_acc[w][g][dim], o);
        L = __builtin_fmaf(f, s_l[w][g], L);
      }
    }
    const int64_t rec = (int64_t)(bh0 + g) * S + s;
    Opart[rec * D + dim] = o;
    if (dim == 0) {
      ML[rec * 2] = (M == -INFINITY) ? -INFINITY : M * kLn2;
      ML[rec * 2 + 1] = L;
    }
  }
}

// Decode split over an FP8 KV cache: K and V rows are OCP E4M3 codes (one byte per element)
// with one float scale per (batch, K/V head), the value of a code being its E4M3 value times the
// scale (KV-cache quantisation, which the Day-21 page's FAQ Q5 names among the decode-side
// techniques: the cache is read with half the bytes of bf16).  Same structure as
// decode_split_kernel: D/16 lanes share a key row (16 codes per lane, one 16-byte load), widened to
// fp32 two at a time by v_cvt_pk_f32_fp8; the K scale is folded into q once and the V scale into
// the partial output.  Queries are bf16 and the partials fp32, so fa_decode_combine is unchanged.
template <int D, int GE>
__global__ __launch_bounds__(256) void decode_split_fp8_kernel(const uint16_t* __restrict__ Q,
                                                               const uint8_t* __restrict__ K,
                                                               const uint8_t* __restrict__ V,
                                                               const float* __restrict__ Ks,
                                                               const float* __restrict__ Vs,
                                                               float* __restrict__ Opart, float* __restrict__ ML,
                                                               int Nk, int S, int chunk, float sl2, int H, int group) {
  constexpr int EPL = 16;         // codes per lane per key row
  constexpr int LPK = D / EPL;    // lanes per key row
  constexpr int KPW = 64 / LPK;   // key rows per wave per step
  constexpr int U = 4;            // steps in flight per iteration
  constexpr int WAVES = 4;
  __shared__ float s_m[WAVES][GE], s_l[WAVES][GE];
  __shared__ float s_acc[WAVES][GE][D];

  const int s = blockIdx.x % S;
  const int bh0 = (blockIdx.x / S) * GE;
  const int start = s * chunk;
  const int end = min(Nk, start + chunk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int gi = lane / LPK, li = lane % LPK;
  const int kvh = (bh0 / H) * (H / group) + (bh0 % H) / group;
  const float ks = Ks[kvh], vs = Vs[kvh];

  float qv[GE][EPL];
#pragma unroll
  for (int g = 0; g < GE; ++g) {
    const uint16_t* qp = Q + (int64_t)(bh0 + g) * D + li * EPL;
    Elt<uint16_t>::widen(gload16(qp), qv[g]);
    Elt<uint16_t>::widen(gload16(qp + 8), qv[g] + 8);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[g][e] *= ks * sl2;  // K scale and scores in log2 units
  }
  const uint8_t* Kh = K + (int64_t)kvh * Nk * D + li * EPL;
  const uint8_t* Vh = V + (int64_t)kvh * Nk * D + li * EPL;
  auto widen8 = [](u32x4_t r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)r[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)r[i], true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  };

  float m[GE], l[GE], acc[GE][EPL];
#pragma unroll
  for (int g = 0; g < GE; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  for (int base = start + wave * U * KPW; base < end; base += WAVES * U * KPW) {
    u32x4_t kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(base + u * KPW + gi, end - 1);
      kr[u] = stream_load16(Kh + (int64_t)key * D);
      vr[u] = stream_load16(Vh + (int64_t)key * D);
    }
    float sc[U][GE];
    float bm[GE];
#pragma unroll
    for (int g = 0; g < GE; ++g) bm[g] = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      widen8(kr[u], kf);
      const bool in = base + u * KPW + gi < end;
#pragma unroll
      for (int g = 0; g < GE; ++g) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[g][e], kf[e], dot);
        dot = group_sum<LPK>(dot);
        sc[u][g] = in ? dot : -INFINITY;
        bm[g] = fmaxf(bm[g], sc[u][g]);
      }
    }
#pragma unroll
    for (int g = 0; g < GE; ++g) {
      bm[g] = max_over_groups<LPK>(bm[g]);
      const float mnew = fmaxf(m[g], bm[g]);
      const float alpha = fast_exp2(m[g] - mnew);
      m[g] = mnew;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      widen8(vr[u], vf);
#pragma unroll
      for (int g = 0; g < GE; ++g) {
        const float p = fast_exp2(sc[u][g] - m[g]);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = __builtin_fmaf(p, vf[e], acc[g][e]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GE; ++g) {
    l[g] = sum_over_groups<LPK>(l[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = sum_over_groups<LPK>(acc[g][e]);
    if (lane == 0) {
      s_m[wave][g] = m[g];
      s_l[wave][g] = l[g];
    }
    if (gi == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][g][li * EPL + e] = acc[g][e];
    }
  }
  __syncthreads();
  for (int x = tid; x < GE * D; x += 256) {
    const int g = x / D, dim = x % D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) M = fmaxf(M, s_m[w][g]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = fast_exp2(s_m[w][g] - M);
        o = __builtin_fmaf(f, s_acc[w][g][dim], o);
        L = __builtin_fmaf(f, s_l[w][g], L);
      }
    }
    const int64_t rec = (int64_t)(bh0 + g) * S + s;
    Opart[rec * D + dim] = o * vs;
    if (dim == 0) {
      ML[rec * 2] = (M == -INFINITY) ? -INFINITY : M * kLn2;
      ML[rec * 2 + 1] = L;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ Opart,
                                                             const float* __restrict__ ML, T* __restrict__ O,
                                                             float* __restrict__ LSE, int S) {
  const int bh = blockIdx.x;
  const int dim = threadIdx.x;
  const float* ml = ML + (int64_t)bh * S * 2;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, acc = 0.f;
  const float* op = Opart + (int64_t)bh * S * D + dim;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float f = fast_exp2((ml[2 * s] - M) * kLog2e);  // empty split: exp2(-inf) = 0
    L = __builtin_fmaf(f, ml[2 * s + 1], L);
    acc = __builtin_fmaf(f, op[(int64_t)s * D], acc);
  }
  O[(int64_t)bh * D + dim] = Elt<T>::narrow(acc / L);
  if (dim == 0) LSE[bh] = M + fast_log2(L) * kLn2;
}

template <typename T, int D, int GE>
void launch_split(const DecodeSplitArgs& a, int chunk, float sl2, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.B * (a.H / GE) * a.num_splits;
  hipLaunchKernelGGL((decode_split_kernel<T, D, GE>), dim3((unsigned)nblk), dim3(256), 0, stream, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, a.o_part, a.ml, a.Nk, a.num_splits, chunk, sl2, a.H,
                     a.H / a.H_kv);
}

template <int D, int GE>
void launch_split_mfma(const DecodeSplitArgs& a, int chunk, float sl2, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.B * (a.H / GE) * a.num_splits;
  hipLaunchKernelGGL((decode_split_mfma_kernel<D, GE>), dim3((unsigned)nblk), dim3(256), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o_part, a.ml, a.Nk,
                     a.num_splits, chunk, sl2, a.H, a.H / a.H_kv);
}

template <typename T, int D>
void launch_split_d(const DecodeSplitArgs& a, int chunk, float sl2, hipStream_t stream) {
  const int group = a.H / a.H_kv;  // query heads per K/V head; a workgroup takes 4, 2 or 1 of them
  // bf16 with grouped heads: both products on the matrix core
  if constexpr (sizeof(T) == 2) {
    if (group % 4 == 0) return launch_split_mfma<D, 4>(a, chunk, sl2, stream);
    if (group % 2 == 0) return launch_split_mfma<D, 2>(a, chunk, sl2, stream);
  }
  if (group % 4 == 0)
    launch_split<T, D, 4>(a, chunk, sl2, stream);
  else if (group % 2 == 0)
    launch_split<T, D, 2>(a, chunk, sl2, stream);
  else
    launch_split<T, D, 1>(a, chunk, sl2, stream);
}

template <typename T>
hipError_t split_impl(const DecodeSplitArgs& a, hipStream_t stream) {
  const int chunk = (a.Nk + a.num_splits - 1) / a.num_splits;
  const float sl2 = a.scale * kLog2e;
  if (a.d == 128)
    launch_split_d<T, 128>(a, chunk, sl2, stream);
  else
    launch_split_d<T, 64>(a, chunk, sl2, stream);
  return hipGetLastError();
}

template <typename T>
hipError_t combine_impl(const DecodeCombineArgs& a, hipStream_t stream) {
  const unsigned nblk = (unsigned)((int64_t)a.B * a.H);
  if (a.d == 128)
    hipLaunchKernelGGL((decode_combine_kernel<T, 128>), dim3(nblk), dim3(128), 0, stream, a.o_part, a.ml, (T*)a.o,
                       a.lse, a.num_splits);
  else
    hipLaunchKernelGGL((decode_combine_kernel<T, 64>), dim3(nblk), dim3(64), 0, stream, a.o_part, a.ml, (T*)a.o,
                       a.lse, a.num_splits);
  return hipGetLastError();
}

template <int D, int GE>
void launch_split_fp8(const DecodeSplitFp8Args& a, int chunk, float sl2, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.B * (a.H / GE) * a.num_splits;
  hipLaunchKernelGGL((decode_split_fp8_kernel<D, GE>), dim3((unsigned)nblk), dim3(256), 0, stream,
                     (const uint16_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.k_scale, a.v_scale, a.o_part,
                     a.ml, a.Nk, a.num_splits, chunk, sl2, a.H, a.H / a.H_kv);
}

template <int D>
void launch_split_fp8_d(const DecodeSplitFp8Args& a, int chunk, float sl2, hipStream_t stream) {
  const int group = a.H / a.H_kv;
  if (group % 4 == 0)
    launch_split_fp8<D, 4>(a, chunk, sl2, stream);
  else if (group % 2 == 0)
    launch_split_fp8<D, 2>(a, chunk, sl2, stream);
  else
    launch_split_fp8<D, 1>(a, chunk, sl2, stream);
}

}  // namespace

hipError_t launch_decode_split_fp8kv(const DecodeSplitFp8Args& a, hipStream_t stream) {
  const int chunk = (a.Nk + a.num_splits - 1) / a.num_splits;
  const float sl2 = a.scale * kLog2e;
  if (a.d == 128)
    launch_split_fp8_d<128>(a, chunk, sl2, stream);
  else
    launch_split_fp8_d<64>(a, chunk, sl2, stream);
  return hipGetLastError();
}

hipError_t launch_decode_split_bf16(const DecodeSplitArgs& a, hipStream_t stream) { return split_impl<uint16_t>(a, stream); }
hipError_t launch_decode_split_f32(const DecodeSplitArgs& a, hipStream_t stream) { return split_impl<float>(a, stream); }
hipError_t launch_decode_combine_bf16(const DecodeCombineArgs& a, hipStream_t stream) {
  return combine_impl<uint16_t>(a, stream);
}
hipError_t launch_decode_combine_f32(const DecodeCombineArgs& a, hipStream_t stream) {
  return combine_impl<float>(a, stream);
}

// ---- fixed scratch of fa_decode_noalloc, for callers that cannot allocate
// The split partials live in this array instead of a caller's workspace.  Each device that loads
// the library holds its own copy, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (on the host it only names a stand-in): the device address
// is looked up once per device and that address is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t decode_scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);  // two racing first calls store the same address
  }
  *out = p;
  return hipSuccess;
}

}  // namespace fa
