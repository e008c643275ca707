// Backward pass of exact attention for gfx950: dQ, dK, dV from Q, K, V, O, dO and the forward's
// per-row LSE, recomputing the probabilities tile by tile instead of storing them (M4-047 card
// "高效注意力与 FlashAttention", §3 point (c); the Day-21 page "GPU 学习日报 Day 21：
// FlashAttention：GPU Memory Hierarchy 下的 IO 优化", §3.2, notes that a standard implementation
// keeps the N x N probabilities for the backward instead).  For one head:
//     P = exp(scale Q K^T - LSE)  (0 where masked),   dV = P^T dO,   dP = dO V^T,
//     dS = P * (dP - Dr),  Dr_i = dO_i . O_i,         dQ = scale dS K,  dK = scale dS^T Q
// (the chain rule through softmax; Dr_i equals rowsum(P * dP) because O = P V).
//
// Three kernels, all on one stream, with no atomics (the result is bit-reproducible):
//  * bwd_pre_kernel: Dr and LSE in log2 units per query row, into the caller's workspace.
//  * bwd_dq_kernel: query-major and ping-pong like the forward.  Each wave owns 32 queries and
//    streams 32-key K/V tiles through LDS rings (LDS DMA): S^T = K Q^T and dP^T = V dO^T on
//    v_mfma_f32_32x32x16_bf16 with Q^T and dO^T held in VGPRs, then dS^T in VGPRs, then
//    dQ^T += K^T dS^T with K^T read from LDS by the transposing ds_read_b64_tr_b16.  Two groups of
//    four waves alternate: while one issues a tile's products, the other computes its dS.  The
//    accumulator-to-B-operand key order (key_of_row) is the forward's.
//  * bwd_dkdv_kernel: key-major, the mirror image of bwd_dq_kernel.  Each wave (one per SIMD)
//    owns 32 keys, with their K^T and V^T fragments in VGPRs, and streams 32-query tiles of Q,
//    dO, LSE and Dr through LDS: S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16_bf16, then P
//    and dS, then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read by the transposing
//    ds_read_b64_tr_b16.  Query rows are loaded in the key_of_row order, so the accumulators are
//    directly the B operands of the last two products.  With grouped K/V heads the workgroup
//    loops over the query heads that share its K/V head and its dK, dV sum over them.
// Recomputing S and dP in both big kernels costs 7 matrix products instead of 5, and keeps both
// free of the cross-workgroup dQ reduction a single kernel would need.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile_layout.h"

namespace fa {
namespace {

// Work item of this workgroup.  Consecutive workgroups go to the eight XCDs in turn; remapping
// them so that XCD x runs the contiguous item range x * n / 8 .. keeps the items of one head on
// one XCD, where they share that head's tiles in the XCD's L2.
__device__ __forceinline__ int xcd_item() {
  const int g = blockIdx.x, n = gridDim.x;
  return (n % 8 == 0) ? (g % 8) * (n / 8) + g / 8 : g;
}

// ------------------------------------------------------------------ preprocess
// One 16-lane group per query row: Dr = dO . O (fp32 sum of bf16 products), L2 = LSE * log2 e.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ LSE, float* __restrict__ L2,
                                                      float* __restrict__ Dr, int64_t rows) {
  constexpr int LPR = 16, EPL = D / LPR;  // lanes per row, elements per lane (8 or 4)
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int li = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const uint16_t* op = O + row * D + li * EPL;
    const uint16_t* dp = dO + row * D + li * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf(bf16_bits_to_f32(op[e]), bf16_bits_to_f32(dp[e]), acc);
  }
#pragma unroll
  for (int w = 1; w < LPR; w <<= 1) acc += __shfl_xor(acc, w);
  if (row < rows && li == 0) {
    Dr[row] = acc;
    L2[row] = LSE[row] * kLog2e;
  }
}

// ------------------------------------------------------------------ dQ
// Query-major, ping-pong like the forward: eight waves in two groups of four, each SIMD running
// one wave of each group.  Workgroup barriers cut time into half-periods; in each, one group
// issues the matrix products of a tile while the other turns its S and dP into dS on the VALU.
// Per 32-key tile t and wave (32 queries):
//   MFMA phase t: S_t^T = K_t Q^T and dP_t^T = V_t dO^T, then dQ^T += K_{t-1}^T dS_{t-1}^T, with
//                 the A operands read from LDS a few MFMAs ahead;
//   VALU phase t: dS_t^T = P_t^T * (dP_t^T - Dr), P = exp2(S sl2 - L2), packed to bf16.
// Group g runs MFMA phase t in half-period 2t + g and VALU phase t in 2t + g + 1.  K_t is read
// in four half-periods (as rows for S by both groups, then transposed for dQ by both) and V_t in
// two, so K tiles sit in a four-slot ring and V tiles in a two-slot ring; group 0 loads tile t + 1
// inside its MFMA phase t, two half-periods before its first use.
template <int D>
struct DqCfg {
  static constexpr int WAVES = 8;  // two groups of four, one wave of each per SIMD
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BR = WAVES * 32;  // queries per workgroup
  static constexpr int BC = 32;          // keys per tile
  static constexpr int RB = D * 2;       // bytes per LDS row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * RB;
  static constexpr int ROWS_PER_DMA = 64 / CPR;
  static constexpr int DMAS = TILE_BYTES / 1024;           // per tensor and tile
  static constexpr int LOADERS = 4;                        // the waves of group 0 move the tiles
  static constexpr int DMA_PER_WAVE = 2 * DMAS / LOADERS;  // K and V together
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int NS = 2 * KSTEPS;  // S and dP MFMAs per tile
  static constexpr int N = NS + 2 * DBLK;  // and the dQ MFMAs
  static_assert(DMAS % LOADERS == 0, "each loading wave moves whole K and V parts");
};

#ifndef FA_DQ_LOOKAHEAD
#define FA_DQ_LOOKAHEAD 6  // MFMAs by which the dQ kernel's LDS operand reads run ahead
#endif

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dr,
    uint16_t* __restrict__ dQ, int H, int group, int Nq, int Nk, int n_qblk, float scale, float sl2, int diag) {
  using C = DqCfg<D>;
  // One array per ring slot, so that the compiler sees the loads into one slot never alias the
  // reads of another.
  __shared__ __attribute__((aligned(1024))) char k0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k2[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k3[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[C::TILE_BYTES];
  auto kslot = [&](auto I) -> char* {
    constexpr int i = decltype(I)::value % 4;
    if constexpr (i == 0) return k0;
    else if constexpr (i == 1) return k1;
    else if constexpr (i == 2) return k2;
    else return k3;
  };
  auto vslot = [&](auto I) -> char* {
    if constexpr (decltype(I)::value % 2 == 0) return v0;
    else return v1;
  };

  // heaviest query blocks first (causal), each head's blocks together
  const int item = xcd_item();
  const int qblk = CAUSAL ? n_qblk - 1 - item % n_qblk : item % n_qblk;
  const int bh = item / n_qblk;
  const int kvh = (bh / H) * (H / group) + (bh % H) / group;
  const uint16_t* Kh = K + (int64_t)kvh * Nk * D;
  const uint16_t* Vh = V + (int64_t)kvh * Nk * D;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int q_wave0 = qblk * C::BR + wave * 32;
  const int q = q_wave0 + l32;
  const int qc = min(q, Nq - 1);

  // Q^T and dO^T fragments (B operands), resident for the whole block
  bf16x8_t qf[C::KSTEPS], dof[C::KSTEPS];
  {
    const uint16_t* qp = Q + ((int64_t)bh * Nq + qc) * D + 8 * hh;
    const uint16_t* dp = dO + ((int64_t)bh * Nq + qc) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      qf[ks] = as_bf16x8(gload16(qp + 16 * ks));
      dof[ks] = as_bf16x8(gload16(dp + 16 * ks));
    }
  }
  const float l2 = L2[(int64_t)bh * Nq + qc];
  const float dr = Dr[(int64_t)bh * Nq + qc];

  const int kv_end = CAUSAL ? min(Nk, qblk * C::BR + C::BR + diag) : Nk;
  const int n = (kv_end + C::BC - 1) / C::BC;

  // Load d (0 <= d < DMA_PER_WAVE) of a loading wave for tile t: the first half of its loads move
  // parts of K, the second half the same parts of V; lane L lands in row L / CPR, slot L % CPR of
  // the part's rows and fetches the chunk the swizzle puts there.  A tile past the last (the load
  // that runs ahead of the block's end) reloads the last one, harmlessly, into a free slot.
  const __amdgpu_buffer_rsrc_t Kr = raw_rsrc(Kh, Nk * C::RB), Vr = raw_rsrc(Vh, Nk * C::RB);
  auto issue_one = [&](int t, int d, char* kdst, char* vdst) {
    constexpr int HALF = C::DMA_PER_WAVE / 2;
    const int c = wave + C::LOADERS * (d % HALF);
    const int row = c * C::ROWS_PER_DMA + lane / C::CPR;
    const int tt = min(t, n - 1);
    const uint32_t off = (uint32_t)min(tt * C::BC + row, Nk - 1) * C::RB + (((lane % C::CPR) ^ swz<D>(row)) << 4);
    char* dst = (d < HALF ? kdst : vdst) + c * 1024;
#if FA_DEBUG_POISON_LDS
    poison16((FA_LDS char*)(dst + lane * 16), kPoisonBf16);
    poison_done();
#endif
    if (d < HALF)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Kr, (lptr_t)dst, 16, off, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Vr, (lptr_t)dst, 16, off, 0, 0, 0);
  };

  // per-lane LDS offsets: 16-byte row reads of permuted keys (A of S^T and dP^T) and transposing
  // 8-byte reads of K^T (A of dQ^T)
  int koff[C::KSTEPS];
  {
    const int krow = key_of_row(l32);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) koff[ks] = krow * C::RB + (((2 * ks + hh) ^ swz<D>(krow)) << 4);
  }
  int toff[C::DBLK][2];
  {
    const int g = lane >> 4, s = lane & 15;
    const int vh = g >> 1, ve = s >> 2, vq = s & 3;
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int key = 8 * vh + 4 * I + ve;
        const int dim = 32 * mb + 16 * (g & 1) + 4 * vq;
        toff[mb][I] = key * C::RB + (((dim >> 3) ^ swz<D>(key)) << 4) + ((dim >> 2) & 1) * 8;
      }
  }

  f32x16_t dq[C::DBLK];
#pragma unroll
  for (int mb = 0; mb < C::DBLK; ++mb) dq[mb] = f32x16_t{};
  f32x16_t s = f32x16_t{}, dp = f32x16_t{};  // S^T and dP^T of the wave's current tile
  u32x4_t dsb[2];                             // bf16 dS^T of the previous tile, two 16-key groups

  // MFMA phase t with K_t in K slot KS (K_{t-1} in KS - 1) and V_t in V slot VS: the S / dP
  // products (DO_S) and dQ of tile t - 1 (DO_DQ), written as an explicit pipeline: slot i issues
  // MFMA i, then the LDS reads of the A operand of MFMA i + L into a rotating set of L + 1
  // registers, and (group 0, LOAD) every few slots one load of tile t + 1 into K slot KS + 1 and
  // V slot VS + 1.  Scheduling barriers between the slots keep the read-ahead.
  auto mfma_phase = [&](int t, auto KSc, auto VSc, auto DO_S, auto DO_DQ, auto LOAD, const char* kprev) {
    constexpr int KS = decltype(KSc)::value, VS = decltype(VSc)::value;
    constexpr int L = FA_DQ_LOOKAHEAD;
    constexpr int i0 = decltype(DO_S)::value ? 0 : C::NS, i1 = decltype(DO_DQ)::value ? C::N : C::NS;
    constexpr int NDMA = decltype(LOAD)::value ? C::DMA_PER_WAVE : 0;
    constexpr int EVERY = (i1 - i0) / (NDMA > 0 ? NDMA : 1);
    const FA_LDS char* kt = (const FA_LDS char*)kslot(std::integral_constant<int, KS>{});
    const FA_LDS char* vt = (const FA_LDS char*)vslot(std::integral_constant<int, VS>{});
    const FA_LDS char* kp = (const FA_LDS char*)kprev;  // K_{t-1}
    char* kdst = kslot(std::integral_constant<int, KS + 1>{});
    char* vdst = vslot(std::integral_constant<int, VS + 1>{});
    bf16x8_t fr[L + 1];
    auto read = [&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < C::NS) {
        fr[i % (L + 1)] = as_bf16x8(lds_load16(((i & 1) ? vt : kt) + koff[i >> 1]));
      } else {
        constexpr int c = i - C::NS, t2 = c / C::DBLK, mb = c % C::DBLK;
        const i16x4_t lo = lds_load8_tr16(kp + toff[mb][0] + t2 * 16 * C::RB);
        const i16x4_t hi = lds_load8_tr16(kp + toff[mb][1] + t2 * 16 * C::RB);
        fr[i % (L + 1)] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    if constexpr (decltype(DO_S)::value) {
      s = f32x16_t{};
      dp = f32x16_t{};
    }
    static_for<L>([&](auto I) {
      if constexpr (i0 + decltype(I)::value < i1) read(std::integral_constant<int, i0 + decltype(I)::value>{});
    });
    static_for<C::N>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i >= i0 && i < i1) {
        if constexpr (i < C::NS) {
          if constexpr (i & 1)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % (L + 1)], dof[i >> 1], dp, 0, 0, 0);
          else
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % (L + 1)], qf[i >> 1], s, 0, 0, 0);
        } else {
          constexpr int c = i - C::NS, t2 = c / C::DBLK, mb = c % C::DBLK;
          dq[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % (L + 1)], as_bf16x8(dsb[t2]), dq[mb], 0, 0, 0);
        }
        if constexpr (i + L < i1) read(std::integral_constant<int, i + L>{});
        if constexpr (NDMA > 0 && (i - i0) % EVERY == 0 && (i - i0) / EVERY < NDMA)
          issue_one(t + 1, (i - i0) / EVERY, kdst, vdst);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    // keep the products in this phase (the next phase would otherwise absorb them)
    asm volatile("" : "+v"(s), "+v"(dp));
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb) asm volatile("" : "+v"(dq[mb]));
  };

  // VALU phase t: P^T and dS^T of the wave's tile; register j of lane-half hh holds key
  // 16 (j / 8) + 8 hh + j % 8 of the tile.  Only tiles past the wave's diagonal or the end of the
  // keys are masked element by element.
  auto valu_phase = [&](int t) {
    const int tile0 = t * C::BC;
    const bool need_mask = (tile0 + C::BC > Nk) || (CAUSAL && tile0 + C::BC - 1 > q_wave0 + diag);
    auto ds_tile = [&](auto mask_tag) {
      const int lim = CAUSAL ? min(Nk - 1, q + diag) : Nk - 1;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float v2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = 8 * t2 + 2 * u + e;
            float p = fast_exp2(__builtin_fmaf(s[j], sl2, -l2));
            if constexpr (decltype(mask_tag)::value) {
              if (tile0 + 16 * t2 + 8 * hh + 2 * u + e > lim) p = 0.f;
            }
            v2[e] = p * (dp[j] - dr);
          }
          dsb[t2][u] = pack_bf16x2(v2[0], v2[1]);
        }
    };
    if (need_mask)
      ds_tile(std::true_type{});
    else
      ds_tile(std::false_type{});
    asm volatile("" : "+v"(dsb[0]), "+v"(dsb[1]));
  };

  auto bar = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
  constexpr std::true_type Y{};
  constexpr std::false_type F{};
  constexpr std::integral_constant<int, 0> I0{};
  constexpr std::integral_constant<int, 1> I1{};
  constexpr std::integral_constant<int, 2> I2{};
  constexpr std::integral_constant<int, 3> I3{};
  // K slot of tile KS - 1
  auto kprev = [&](auto KSc) -> const char* { return kslot(std::integral_constant<int, decltype(KSc)::value + 3>{}); };
  // the last MFMA phase (tile n: dQ of tile n - 1 only), with K_{n-1} in K slot (n - 1) mod 4
  auto last_dq = [&]() {
    const int r = (n - 1) & 3;
    const char* kl = r == 0 ? k0 : r == 1 ? k1 : r == 2 ? k2 : k3;
    mfma_phase(n, I0, I0, F, Y, F, kl);
  };

  if (grp == 0) {
#pragma unroll
    for (int d = 0; d < C::DMA_PER_WAVE; ++d) issue_one(0, d, k0, v0);
  }
  wait_loads();
  bar();
  if (grp == 0) {
    mfma_phase(0, I0, I0, Y, F, Y, k3);  // h = 0: S_0, dP_0; loads tile 1
    bar();
    valu_phase(0);  // h = 1
    wait_loads();
    bar();
    // tile t: MFMA phase in half-period 2t, VALU phase in 2t + 1
    auto both = [&](int t, auto KSc, auto VSc) {
      mfma_phase(t, KSc, VSc, Y, Y, Y, kprev(KSc));
      bar();
      valu_phase(t);
      wait_loads();
      bar();
    };
    int t = 1;
    for (; t + 3 < n; t += 4) {
      both(t, I1, I1);
      both(t + 1, I2, I0);
      both(t + 2, I3, I1);
      both(t + 3, I0, I0);
    }
    if (t < n) both(t, I1, I1);
    if (t + 1 < n) both(t + 1, I2, I0);
    if (t + 2 < n) both(t + 2, I3, I1);
    last_dq();  // h = 2n
    bar();
  } else {
    bar();                           // h = 0: idle
    mfma_phase(0, I0, I0, Y, F, F, k3);  // h = 1
    bar();
    // tile t: VALU phase of tile t - 1 in half-period 2t, MFMA phase of tile t in 2t + 1
    auto both = [&](int t, auto KSc, auto VSc) {
      valu_phase(t - 1);
      bar();
      mfma_phase(t, KSc, VSc, Y, Y, F, kprev(KSc));
      bar();
    };
    int t = 1;
    for (; t + 3 < n; t += 4) {
      both(t, I1, I1);
      both(t + 1, I2, I0);
      both(t + 2, I3, I1);
      both(t + 3, I0, I0);
    }
    if (t < n) both(t, I1, I1);
    if (t + 1 < n) both(t + 1, I2, I0);
    if (t + 2 < n) both(t + 2, I3, I1);
    valu_phase(n - 1);  // h = 2n
    bar();
    last_dq();  // h = 2n + 1
  }

  if (q < Nq) {
    uint16_t* op = dQ + ((int64_t)bh * Nq + q) * D + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        u32x2_t w;
        w[0] = pack_bf16x2(dq[mb][4 * jg + 0] * scale, dq[mb][4 * jg + 1] * scale);
        w[1] = pack_bf16x2(dq[mb][4 * jg + 2] * scale, dq[mb][4 * jg + 3] * scale);
        *(u32x2_t*)(op + 32 * mb + 8 * jg) = w;
      }
  }
}

// ------------------------------------------------------------------ dK, dV
#ifndef FA_BWD_LOOKAHEAD
#define FA_BWD_LOOKAHEAD 3  // MFMAs by which the dK/dV kernel's LDS operand reads run ahead
#endif

// Key-major, one wave per SIMD: each wave owns 32 keys, so that every 16-byte LDS operand read
// feeds a 32x32x16 MFMA (32 keys x 32 queries x 16) and the Q and dO tiles, read twice per wave
// (as rows for S and dP, transposed for dK and dV), cost one LDS byte per 32 FLOP.  The 32-key
// accumulators of dK^T and dV^T with the K and V fragments take more registers than two waves
// per SIMD have, so the wave overlaps its own work: while the matrix core computes S and dP of
// the next query tile, the VALU turns the current tile's S and dP into P and dS.
template <int D>
struct DkvCfg {
  static constexpr int WAVES = 4;        // one per SIMD
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BK = WAVES * 32;  // keys per workgroup, 32 per wave
  static constexpr int BQ = 32;          // queries per tile
  static constexpr int SLOTS = 3;        // LDS ring: the tile in use, the next, one loading
  static constexpr int RB = D * 2;       // bytes per LDS row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int TILE_BYTES = BQ * RB;
  static constexpr int ROWS_PER_DMA = 64 / CPR;
  static constexpr int DMAS = TILE_BYTES / 1024;         // per tensor and tile
  static constexpr int DMA_PER_WAVE = 2 * DMAS / WAVES;  // Q and dO together
  static constexpr int KSTEPS = D / 16;                  // k-steps of S = Q K^T
  static constexpr int DBLK = D / 32;                    // 32-dim blocks of dK^T, dV^T
  static_assert((2 * DMAS) % WAVES == 0, "tile loads must split evenly over the waves");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws, int64_t rows_total,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int H, int group, int Nq, int Nk, int n_kblk,
    float scale, float sl2, int diag) {
  using C = DkvCfg<D>;
  // One array per slot and tensor: the compiler then tells a slot being read from the one a load is
  // filling, and waits for a tile's loads only where that tile is read.  All of them lie below
  // 64 KiB, in reach of the ds_read immediate offset.
  __shared__ __attribute__((aligned(1024))) char q0b[C::TILE_BYTES], q1b[C::TILE_BYTES], q2b[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char o0b[C::TILE_BYTES], o1b[C::TILE_BYTES], o2b[C::TILE_BYTES];
  __shared__ __attribute__((aligned(256))) float s0b[2 * C::BQ], s1b[2 * C::BQ], s2b[2 * C::BQ];  // [L2][Dr]
  auto qslot = [&](auto I) -> char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return q0b;
    else if constexpr (i == 1) return q1b;
    else return q2b;
  };
  auto oslot = [&](auto I) -> char* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return o0b;
    else if constexpr (i == 1) return o1b;
    else return o2b;
  };
  auto sslot = [&](auto I) -> float* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return s0b;
    else if constexpr (i == 1) return s1b;
    else return s2b;
  };

  const int item = xcd_item();
  const int kblk = item % n_kblk;
  const int bkv = item / n_kblk;  // b * H_kv + kv head
  const int H_kv = H / group;
  const int b = bkv / H_kv, hk = bkv % H_kv;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k0 = kblk * C::BK;
  const int kw0 = k0 + wave * 32;  // the wave's first key
  const int key = kw0 + l32;       // this lane's key (column of every accumulator)
  const int keyc = min(key, Nk - 1);

  // K^T and V^T fragments (B operands of S and dP): key `key`, dims 16 ks + 8 hh .. + 7
  bf16x8_t kf[C::KSTEPS], vf[C::KSTEPS];
  {
    const uint16_t* kp = K + ((int64_t)bkv * Nk + keyc) * D + 8 * hh;
    const uint16_t* vp = V + ((int64_t)bkv * Nk + keyc) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      kf[ks] = as_bf16x8(gload16(kp + 16 * ks));
      vf[ks] = as_bf16x8(gload16(vp + 16 * ks));
      // only ever MFMA operands: kept in the accumulation registers, leaving the VGPRs to the
      // two tiles of S and dP the VALU works on
      asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));
    }
  }

  // LDS offsets.  S and dP: MFMA row m reads query key_of_row(m) of the tile, so register j of
  // lane-half hh of S and dP is query 16 (j / 8) + 8 hh + j % 8 and 8 consecutive registers,
  // packed to bf16, are the B operand (k = those queries) of dV^T and dK^T.  Their A operands,
  // dO^T and Q^T, come from the transposing ds_read_b64_tr_b16: lane l receives dim
  // 32 mb + l % 32 of queries 16 t2 + 8 hh .. + 7 (t2 the k-step).
  int roff[C::KSTEPS];
  {
    const int qrow = key_of_row(l32);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) roff[ks] = qrow * C::RB + (((2 * ks + hh) ^ swz<D>(qrow)) << 4);
  }
  int toff[C::DBLK][2];
  {
    const int g = lane >> 4, s = lane & 15;
    const int vh = g >> 1, ve = s >> 2, vq = s & 3;
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int row = 8 * vh + 4 * I + ve;
        const int dim = 32 * mb + 16 * (g & 1) + 4 * vq;
        toff[mb][I] = row * C::RB + (((dim >> 3) ^ swz<D>(row)) << 4) + ((dim >> 2) & 1) * 8;
      }
  }

  f32x16_t dk[C::DBLK], dv[C::DBLK];
#pragma unroll
  for (int mb = 0; mb < C::DBLK; ++mb) {
    dk[mb] = f32x16_t{};
    dv[mb] = f32x16_t{};
  }

  // query tiles this workgroup's keys can be seen from: query i sees key j iff j <= i + diag;
  // they are visited from the last one down, so that the workgroups of one head (all on one XCD)
  // read the same tile at about the same time whatever their first tile
  const int q_first = CAUSAL ? max(0, k0 - diag) / C::BQ : 0;
  const int n_qt = (Nq + C::BQ - 1) / C::BQ;
  const int n_steps = n_qt - q_first;
  // the statistics load takes L2 in lanes 0-31 and Dr in lanes 32-63
  const int stat_off = (int)((hh * rows_total + l32) * 4);

  auto bar = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // wait until at most n of this wave's vector memory loads are outstanding
  auto wait_loads_but = [&](auto N) {
    constexpr int n = decltype(N)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70 | n);
  };

  f32x16_t S[2], DP[2];  // S and dP of two tiles: the one the VALU consumes, the one the MFMAs fill
  u32x4_t pB[2], dsB[2];

  for (int gh = 0; gh < group; ++gh) {
    if (n_steps <= 0) break;
    const int bh = b * H + hk * group + gh;  // query head
    const uint16_t* Qh = Q + (int64_t)bh * Nq * D;
    const uint16_t* Oh = dO + (int64_t)bh * Nq * D;
    // Tile t's loads, each tensor through a buffer resource based at the tile's first row with its
    // range ending at the head's last row (the statistics': at the workspace's end), so a lane's
    // offset is the same for every tile and rows past the last query read as zero.  Instruction i
    // of this wave moves 1 KiB of Q (x < DMAS) or dO, lane L landing in row L / CPR, slot L % CPR
    // of the instruction's rows and fetching the chunk the swizzle puts there.  The last wave also
    // moves the statistics.
    auto issue = [&](int t, auto SLOT) {
      const int r0 = t * C::BQ;
      const __amdgpu_buffer_rsrc_t Qr = raw_rsrc(Qh + (int64_t)r0 * D, (Nq - r0) * C::RB);
      const __amdgpu_buffer_rsrc_t Or = raw_rsrc(Oh + (int64_t)r0 * D, (Nq - r0) * C::RB);
#pragma unroll
      for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
        const int x = wave + C::WAVES * i;
        const int c = x % C::DMAS;
        const int row = c * C::ROWS_PER_DMA + lane / C::CPR;
        const int off = row * C::RB + (((lane % C::CPR) ^ swz<D>(row)) << 4);
        if (x < C::DMAS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(Qr, (lptr_t)(qslot(SLOT) + c * 1024), 16, off, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(Or, (lptr_t)(oslot(SLOT) + c * 1024), 16, off, 0, 0, 0);
      }
      if (wave == C::WAVES - 1) {
        const int64_t e0 = (int64_t)bh * Nq + r0;
        const __amdgpu_buffer_rsrc_t Sr = raw_rsrc(ws + e0, (int)((2 * rows_total - e0) * 4));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(Sr, (lptr_t)sslot(SLOT), 4, stat_off, 0, 0, 0);
      }
    };
    auto tile_of = [&](int k) { return n_qt - 1 - k; };

    // One step: the S / dP MFMAs of tile k + 1 (slot SN, into set 1 - RC) with P and dS of tile
    // k (set RC, statistics of slot SC) on the VALU between them, then dV^T += dO^T P and
    // dK^T += Q^T dS from tile k's slot.  MFMA i < 16 is k-step i / 2 of S (even) or dP (odd);
    // MFMA 16 + i is k-step t2 = i / (2 DBLK) of dim block (i / 2) % DBLK, dV (even) or dK.
    // Every operand read runs LA MFMAs ahead.  The last step computes S and dP of a stale slot
    // and drops them, so that every step has the same schedule.
    auto body = [&](auto SC, auto SN, auto RC) {
      constexpr int rc = decltype(RC)::value, rn = 1 - rc;
      constexpr int LA = FA_BWD_LOOKAHEAD, NA = 2 * C::KSTEPS, NC = 4 * C::DBLK, N = NA + NC;
      const FA_LDS char* qn = (const FA_LDS char*)qslot(SN);
      const FA_LDS char* on = (const FA_LDS char*)oslot(SN);
      const FA_LDS char* qc = (const FA_LDS char*)qslot(SC);
      const FA_LDS char* oc = (const FA_LDS char*)oslot(SC);
      const FA_LDS float* st = (const FA_LDS float*)sslot(SC);
      u32x4_t fr[LA + 1];
      auto read = [&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i < NA) {
          fr[i % (LA + 1)] = lds_load16(((i & 1) ? on : qn) + roff[i >> 1]);
        } else {
          constexpr int c = i - NA, t2 = c / (2 * C::DBLK), mb = (c >> 1) % C::DBLK;
          const FA_LDS char* base = ((c & 1) ? qc : oc) + t2 * 16 * C::RB;
          const i16x4_t lo = lds_load8_tr16(base + toff[mb][0]);
          const i16x4_t hi = lds_load8_tr16(base + toff[mb][1]);
          fr[i % (LA + 1)] = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      // P and dS of tile k in eight units of two elements (unit w: j = 2 w, 2 w + 1, queries
      // 16 t2 + 8 hh + 2 u + e), each in four stages one MFMA slot apart, so that no slot waits for
      // a result of its own: A the exponent and dP - Dr, B the exponentials, C dS and the packed
      // P, D the packed dS.  Unit w starts at slot G w; its L2 and Dr are read three slots earlier.
      typedef float f32x2_t __attribute__((ext_vector_type(2)));
      constexpr int G = NA / 8;
      f32x2_t l2u[8], dru[8], ta[8], da[8], pa[8], dsa[8];
      auto stats = [&](auto W) {
        constexpr int w = decltype(W)::value, t2 = w >> 2, u = w & 3;
        l2u[w] = *(const FA_LDS f32x2_t*)(st + 16 * t2 + 8 * hh + 2 * u);
        dru[w] = *(const FA_LDS f32x2_t*)(st + C::BQ + 16 * t2 + 8 * hh + 2 * u);
      };
      auto stage = [&](auto W, auto X) {
        constexpr int w = decltype(W)::value, x = decltype(X)::value, t2 = w >> 2, u = w & 3, j = 8 * t2 + 2 * u;
        if constexpr (x == 0) {
          ta[w][0] = __builtin_fmaf(S[rc][j], sl2, -l2u[w][0]);
          ta[w][1] = __builtin_fmaf(S[rc][j + 1], sl2, -l2u[w][1]);
          da[w][0] = DP[rc][j] - dru[w][0];
          da[w][1] = DP[rc][j + 1] - dru[w][1];
        } else if constexpr (x == 1) {
          pa[w][0] = fast_exp2(ta[w][0]);
          pa[w][1] = fast_exp2(ta[w][1]);
        } else if constexpr (x == 2) {
          dsa[w][0] = pa[w][0] * da[w][0];
          dsa[w][1] = pa[w][1] * da[w][1];
          pB[t2][u] = pack_bf16x2(pa[w][0], pa[w][1]);
        } else {
          dsB[t2][u] = pack_bf16x2(dsa[w][0], dsa[w][1]);
        }
      };
      // the work of slot i (i = -1: before the first MFMA)
      auto valu_slot = [&](auto I) {
        constexpr int i = decltype(I)::value;
        static_for<8>([&](auto W) {
          constexpr int w = decltype(W)::value, s0 = G * w;
          if constexpr ((s0 - 3 < 0 ? -1 : s0 - 3) == i) stats(W);
          static_for<4>([&](auto X) {
            if constexpr (s0 + decltype(X)::value == i) stage(W, X);
          });
        });
      };
      S[rn] = f32x16_t{};
      DP[rn] = f32x16_t{};
      valu_slot(std::integral_constant<int, -1>{});
      static_for<LA>([&](auto I) { read(I); });
      static_for<N>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i < NA) {
          if constexpr (i & 1)
            DP[rn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[i % (LA + 1)]), vf[i >> 1], DP[rn], 0, 0, 0);
          else
            S[rn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[i % (LA + 1)]), kf[i >> 1], S[rn], 0, 0, 0);
        } else {
          constexpr int c = i - NA, t2 = c / (2 * C::DBLK), mb = (c >> 1) % C::DBLK;
          if constexpr (c & 1)
            dk[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[i % (LA + 1)]), as_bf16x8(dsB[t2]), dk[mb], 0, 0, 0);
          else
            dv[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[i % (LA + 1)]), as_bf16x8(pB[t2]), dv[mb], 0, 0, 0);
        }
        if constexpr (i + LA < N) read(std::integral_constant<int, i + LA>{});
        valu_slot(I);
        __builtin_amdgcn_sched_barrier(0);
      });
      asm volatile("" : "+v"(S[rn]), "+v"(DP[rn]));
    };

    // Step k (tile k is in slot k % 3 and its S / dP in set k % 2): wait for tile k + 1, meet the
    // other waves (all past step k - 1, so the slot of tile k - 1 is free), start tile k + 2 into
    // it, then the body.
    auto step = [&](int k, auto P) {
      constexpr int p = decltype(P)::value;
      wait_loads_but(std::integral_constant<int, 0>{});
      bar();
      if (k + 2 < n_steps) {
        constexpr std::integral_constant<int, (p + 2) % C::SLOTS> SL{};
#if FA_DEBUG_POISON_LDS
        {  // the slot of tile k - 1, retired by this barrier
#pragma unroll
          for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
            const int x = wave + C::WAVES * i;
            poison16((FA_LDS char*)((x < C::DMAS ? qslot(SL) : oslot(SL)) + (x % C::DMAS) * 1024 + lane * 16), kPoisonBf16);
          }
          if (wave == C::WAVES - 1) *((FA_LDS uint32_t*)sslot(SL) + lane) = kPoisonF32;
          poison_done();
        }
#endif
        issue(tile_of(k + 2), SL);
      }
      // a tile that reaches past the wave's diagonal or the end of the queries: its masked
      // scores become -inf, so that P and dS are 0 there
      const int q0 = tile_of(k) * C::BQ;
      if ((q0 + C::BQ > Nq) || (CAUSAL && kw0 + 31 > q0 + diag)) {
        constexpr int rc = p % 2;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int qq = q0 + 16 * (j >> 3) + 8 * hh + (j & 7);
          if (qq >= Nq || (CAUSAL && key > qq + diag)) S[rc][j] = -INFINITY;
        }
      }
      body(std::integral_constant<int, p % C::SLOTS>{}, std::integral_constant<int, (p + 1) % C::SLOTS>{},
           std::integral_constant<int, p % 2>{});
    };

    // prologue: tiles 0 and 1 into slots 0 and 1 (after every wave has left the previous head's
    // slots), and S / dP of tile 0 into set 0
    bar();
    issue(tile_of(0), std::integral_constant<int, 0>{});
    if (n_steps > 1) issue(tile_of(1), std::integral_constant<int, 1>{});
    wait_loads_but(std::integral_constant<int, 0>{});
    bar();
    {
      constexpr int LA = FA_BWD_LOOKAHEAD, NA = 2 * C::KSTEPS;
      const FA_LDS char* q0t = (const FA_LDS char*)q0b;
      const FA_LDS char* o0t = (const FA_LDS char*)o0b;
      u32x4_t fr[LA + 1];
      auto read = [&](auto I) {
        constexpr int i = decltype(I)::value;
        fr[i % (LA + 1)] = lds_load16(((i & 1) ? o0t : q0t) + roff[i >> 1]);
      };
      S[0] = f32x16_t{};
      DP[0] = f32x16_t{};
      static_for<LA>([&](auto I) { read(I); });
      static_for<NA>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i & 1)
          DP[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[i % (LA + 1)]), vf[i >> 1], DP[0], 0, 0, 0);
        else
          S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fr[i % (LA + 1)]), kf[i >> 1], S[0], 0, 0, 0);
        if constexpr (i + LA < NA) read(std::integral_constant<int, i + LA>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      asm volatile("" : "+v"(S[0]), "+v"(DP[0]));
    }
    for (int k = 0;;) {
      step(k, std::integral_constant<int, 0>{});
      if (++k >= n_steps) break;
      step(k, std::integral_constant<int, 1>{});
      if (++k >= n_steps) break;
      step(k, std::integral_constant<int, 2>{});
      if (++k >= n_steps) break;
      step(k, std::integral_constant<int, 3>{});
      if (++k >= n_steps) break;
      step(k, std::integral_constant<int, 4>{});
      if (++k >= n_steps) break;
      step(k, std::integral_constant<int, 5>{});
      if (++k >= n_steps) break;
    }
  }

  // dK = scale (dK^T)^T, dV = (dV^T)^T: register 4 jg + i of block mb is dim 32 mb + 8 jg + 4 hh + i
  if (key < Nk) {
    uint16_t* kp = dK + ((int64_t)bkv * Nk + key) * D + 4 * hh;
    uint16_t* vp = dV + ((int64_t)bkv * Nk + key) * D + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        u32x2_t wk, wv;
        wk[0] = pack_bf16x2(dk[mb][4 * jg + 0] * scale, dk[mb][4 * jg + 1] * scale);
        wk[1] = pack_bf16x2(dk[mb][4 * jg + 2] * scale, dk[mb][4 * jg + 3] * scale);
        wv[0] = pack_bf16x2(dv[mb][4 * jg + 0], dv[mb][4 * jg + 1]);
        wv[1] = pack_bf16x2(dv[mb][4 * jg + 2], dv[mb][4 * jg + 3]);
        *(u32x2_t*)(kp + 32 * mb + 8 * jg) = wk;
        *(u32x2_t*)(vp + 32 * mb + 8 * jg) = wv;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_impl(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.Nq;
  float* L2 = a.ws;
  float* Dr = a.ws + rows;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                     (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, L2, Dr, rows);
  const float sl2 = a.scale * kLog2e;
  const int group = a.H / a.H_kv;
  {
    using C = DqCfg<D>;
    const int n_qblk = (a.Nq + C::BR - 1) / C::BR;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)a.B * a.H * n_qblk)), dim3(C::THREADS),
                       0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, L2, Dr, (uint16_t*)a.dq, a.H, group, a.Nq, a.Nk, n_qblk, a.scale, sl2,
                       a.diag);
  }
  {
    using C = DkvCfg<D>;
    const int n_kblk = (a.Nk + C::BK - 1) / C::BK;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)a.B * a.H_kv * n_kblk)),
                       dim3(C::THREADS), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, (const float*)a.ws, rows, (uint16_t*)a.dk, (uint16_t*)a.dv, a.H, group,
                       a.Nq, a.Nk, n_kblk, a.scale, sl2, a.diag);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_bwd_impl<128, true>(a, stream) : launch_bwd_impl<128, false>(a, stream);
  return a.causal ? launch_bwd_impl<64, true>(a, stream) : launch_bwd_impl<64, false>(a, stream);
}

}  // namespace fa
