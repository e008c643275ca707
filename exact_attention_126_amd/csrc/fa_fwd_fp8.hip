// Fused attention forward with FP8 inputs for gfx950: Q, K and V are OCP FP8 E4M3 codes with one
// float scale per (batch, head) and tensor; O is bf16, LSE fp32.  The method is the one of
// fa_fwd.hip (Day-21 page "GPU 学习日报 Day 21：FlashAttention：GPU Memory Hierarchy 下的 IO 优化",
// §4 tiling, §5.2-5.3 online softmax), with both products on the FP8 matrix core (the same page
// names FP8 as a FlashAttention-3 feature at the close of its §6).
//
// gfx950 mapping (what differs from the bf16 kernel):
//  * Both products on v_mfma_f32_32x32x64_f8f6f4 (fp8 x fp8, fp32 accumulate), which does four
//    times the k-depth of the bf16 32x32x16 in twice its cycles: S^T = K Q^T takes D/64 k-steps
//    per 32-key block, O^T = V^T P^T one k-step per 64 keys and 32-dim block.  Each operand
//    lane holds 32 bytes (k values) of row or column l % 32; A and B share the k order, which is
//    all the products need.
//  * Codes multiply as codes: S^T is Q_codes K_codes^T, and scale * q_scale * k_scale * log2(e) is
//    one per-head factor in the exponent; v_scale multiplies the output once at the end.
//  * P is rounded to E4M3 (v_cvt_pk_fp8_f32, round to nearest even) for the second product.  To
//    keep small probabilities out of the E4M3 subnormals, P is computed as exp2(s - m + 4) with
//    the running max raised lazily by more than 4 (log2 units): every value stays <= 2^8 (E4M3
//    holds up to 448) and values down to 2^-10 of the row max are normal.  The row sum l is
//    accumulated from the unrounded fp32 P, so the LSE is as accurate as the scores.
//  * K rows are read in natural order.  Register j of accumulator lane-half h holds key row
//    8*(j/4) + 4*h + (j%4) (+32 for the second block), so the 32 P bytes a lane feeds the second
//    product are those keys; the transposing V reads (ds_read_b64_tr_b8) take their row
//    addresses in that order.  Within 16 lanes, lane i of ds_read_b64_tr_b8 receives byte i % 8
//    of the 8-byte pieces addressed by lanes 2e + i/8, e = 0..7.
//  * LDS rows (D bytes) are XOR-swizzled in 16-byte chunks by row bits 1-3, chosen so that the
//    K operand reads and the transposing V reads are free of bank conflicts.
//  * Workgroup shape, ping-pong between two groups of four waves, LDS DMA of the tiles, the
//    persistent balanced grid and the XCD-aware order are those of the bf16 kernel.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

#ifndef FA8_TILE
#define FA8_TILE 128  // keys per tile: with 128 the MFMA phase (16 MFMAs at d = 128) is as long as the
                      // bf16 kernel's, and the barriers and per-tile softmax work per key halve
#endif
#ifndef FA_CAUSAL_SKIP
#define FA_CAUSAL_SKIP 1  // causal: a wave skips the products and softmax of tiles past its diagonal
#endif

template <int D, int BCK = FA8_TILE>
struct Fp8Cfg {
  static constexpr int WAVES = 8;  // two groups of four, one wave of each per SIMD
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BR = WAVES * 32;  // query rows per workgroup, 32 per wave
  static constexpr int BC = BCK;         // keys per tile
  static constexpr int SB = BC / 32;     // 32-key blocks of S^T per tile
  static constexpr int PH = BC / 64;     // 64-key k-steps of O^T += V^T P^T per tile
  static constexpr int RB = D;           // bytes per LDS row
  static constexpr int CPR = D / 16;     // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * RB;
  static constexpr int ROWS_PER_DMA = 64 / CPR;  // rows one wave-wide 1 KiB LDS load fills
  static constexpr int LOADERS = 4;
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / LOADERS;  // per tensor and tile
  static constexpr int KSTEPS = D / 64;                             // k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 32;                               // 32-dim blocks of O^T
  static_assert(TILE_BYTES % (1024 * LOADERS) == 0, "tile must split evenly into wave loads");
};

// Lazy-rescale threshold and exponent offset (log2 units): P = exp2(s - m + kBias) with m raised
// only when a row max exceeds it by more than kTau, so P <= 2^(kTau + kBias) = 256 < 448.
constexpr float kTau = 4.f;
constexpr float kBias = 4.f;

#ifndef FA8_LOOKAHEAD
#define FA8_LOOKAHEAD 3  // MFMAs by which LDS operand reads run ahead
#endif

// 16-byte chunk swizzle of a D-byte LDS row, from row bits 1-3.
template <int D>
__device__ __forceinline__ int swz8(int row);
template <>
__device__ __forceinline__ int swz8<128>(int row) {
  return ((row & 2) ? 2 : 0) ^ ((row & 4) ? 1 : 0) ^ ((row & 8) ? 4 : 0);
}
template <>
__device__ __forceinline__ int swz8<64>(int row) {
  return ((row & 4) ? 1 : 0) ^ ((row & 8) ? 2 : 0);
}

// Key row (within 64 keys of the tile) of byte b (0..31) of the P operand in lane-half h: the
// accumulator row of the S^T register it was converted from.
__device__ __forceinline__ int key_of_pbyte(int b, int h) {
  const int blk = b >> 4, j = b & 15;
  return 32 * blk + 8 * (j >> 2) + 4 * h + (j & 3);
}

__device__ __forceinline__ f32x16_t mfma8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // fp8 (E4M3) x fp8, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8_t join16(u32x4_t lo, u32x4_t hi) {
  return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ i32x2_t lds_load8_tr8(const FA_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2_t*)p);
}

// One query block of the FP8 forward (see fwd_block in fa_fwd.hip for the phase structure,
// which is the same).  sl2 = scale * log2(e) * q_scale * k_scale of this head, vsc = v_scale.
template <int D, bool CAUSAL>
__device__ __forceinline__ void fp8_block(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                          const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
                                          float* __restrict__ LSE, int Nq, int Nk, float sl2, float vsc, int bh,
                                          int kvh, int diag, int qblk, int n_qblk, char* kb0, char* kb1, char* vb0,
                                          char* vb1, char* stg) {
  using C = Fp8Cfg<D>;
  const uint8_t* Qh = Q + (int64_t)bh * Nq * D;
  const uint8_t* Kh = K + (int64_t)kvh * Nk * D;
  const uint8_t* Vh = V + (int64_t)kvh * Nk * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int q_wave0 = qblk * C::BR + wave * 32;
  // Causal: the last tile with a key this wave's rows can see.  Later tiles would give the wave
  // only -inf scores and P = 0, so it skips their products and softmax (the same result bit for bit)
  // and keeps only its part of the barriers and tile loads.
  const int j_last = (CAUSAL && FA_CAUSAL_SKIP) ? (q_wave0 + 31 + diag) / C::BC : 0;

  // ---- Q^T fragments (B operand): query l32, dims 64 ks + 32 hh .. + 31
  i32x8_t qf[C::KSTEPS];
  {
    const int qrow = min(q_wave0 + l32, Nq - 1);
    const uint8_t* qp = Qh + (int64_t)qrow * D + 32 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[ks] = join16(gload16(qp + 64 * ks), gload16(qp + 64 * ks + 16));
  }

  const int kv_end = CAUSAL ? min(Nk, qblk * C::BR + C::BR + diag) : Nk;
  const int n = (kv_end + C::BC - 1) / C::BC;
  const int rot = CAUSAL ? 0 : (int)(((int64_t)qblk * n) / n_qblk);
  auto tile_of = [&](int t) {
    const int x = t + rot;
    return x >= n ? x - n : x;
  };

  // ---- global -> LDS tile loads (group 0, inside its MFMA phases); LDS row = key row of the tile.
  // Each tile gets its own buffer resource (base at the tile's first key, range ending at the
  // head's last key), so a lane's byte offset is the same for every tile and a load costs no
  // vector instruction; rows past the last key are outside the range and read as zero without a
  // memory access (the rings are zero-filled at kernel start as well).
  const int lw = wave & 3;
  int dma_off[C::DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
    const int row = (lw * C::DMA_PER_WAVE + i) * C::ROWS_PER_DMA + lane / C::CPR;
    dma_off[i] = row * C::RB + ((lane % C::CPR) ^ swz8<D>(row)) * 16;
  }
  auto issue_one = [&](const uint8_t* src, int t, char* buf, int i) {
    const int r0 = tile_of(t) * C::BC;
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(src + (int64_t)r0 * C::RB, (Nk - r0) * C::RB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(buf + (lw * C::DMA_PER_WAVE + i) * 1024), 16, dma_off[i], 0, 0, 0);
  };
  auto issue = [&](const uint8_t* src, int t, char* buf) {
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) issue_one(src, t, buf, i);
  };

  // ---- per-lane LDS read offsets.  K: row l32 (+32 for the second block), dims 64 ks + 32 hh.
  int koff[C::KSTEPS][2];
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c) koff[ks][c] = l32 * C::RB + (((4 * ks + 2 * hh + c) ^ swz8<D>(l32)) << 4);
  // V (transposing reads): read r of 32-dim block mb; this lane addresses byte (8r + i'/2) of the
  // P operand of lane-half hh, i.e. key row key_of_pbyte, at dims 32 mb + 16 (g & 1) + 8 (i' & 1).
  int voff[C::DBLK][4];
  {
    const int g = lane >> 4, ip = lane & 15;
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = key_of_pbyte(8 * r + (ip >> 1), hh);
        voff[mb][r] = row * C::RB + (((2 * mb + (g & 1)) ^ swz8<D>(row)) << 4) + 8 * (ip & 1);
      }
  }

  f32x16_t oacc[C::DBLK];
#pragma unroll
  for (int mb = 0; mb < C::DBLK; ++mb) oacc[mb] = f32x16_t{};
  float m2 = -INFINITY, lsum = 0.f;
  f32x16_t sacc[C::SB];  // S^T of the current tile, 32-key blocks
  f32x16_t& s0 = sacc[0];
  f32x16_t& s1 = sacc[1];
  // E4M3 P^T of the previous tile, per 64 keys (32 keys per lane-half).  Zeroed once per block:
  // the packing below reads each word (only to overwrite it half by half), so it must never be
  // indeterminate.
  i32x8_t pb[C::PH];
#pragma unroll
  for (int h = 0; h < C::PH; ++h) pb[h] = i32x8_t{};

  auto kfrag = [&](const FA_LDS char* kt, int blk, int ks) {
    return join16(lds_load16(kt + blk * 32 * C::RB + koff[ks][0]), lds_load16(kt + blk * 32 * C::RB + koff[ks][1]));
  };
  auto vfrag = [&](const FA_LDS char* vt, int mb) {
    const i32x2_t r0 = lds_load8_tr8(vt + voff[mb][0]), r1 = lds_load8_tr8(vt + voff[mb][1]);
    const i32x2_t r2 = lds_load8_tr8(vt + voff[mb][2]), r3 = lds_load8_tr8(vt + voff[mb][3]);
    return i32x8_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  };
  auto qk = [&](const char* kbuf) {
    const FA_LDS char* kt = (const FA_LDS char*)kbuf;
#pragma unroll
    for (int b = 0; b < C::SB; ++b) sacc[b] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int b = 0; b < C::SB; ++b) sacc[b] = mfma8(kfrag(kt, b, ks), qf[ks], sacc[b]);
  };
  auto pv = [&](const char* vbuf) {
    const FA_LDS char* vt = (const FA_LDS char*)vbuf;
#pragma unroll
    for (int h = 0; h < C::PH; ++h)
#pragma unroll
      for (int mb = 0; mb < C::DBLK; ++mb) oacc[mb] = mfma8(vfrag(vt + h * 64 * C::RB, mb), pb[h], oacc[mb]);
  };
  // The tile's largest raw score of this lane's row is taken in the MFMA phase that computes S,
  // under its P V products (sixteen dependent max3 steps, then the swap across the lane halves):
  // the FP8 MFMA phase is half as long as the softmax phase, whose single wave issues a VALU
  // instruction only every few cycles.  Tiles that need an element mask take it again after
  // masking.
  float smax_pre = 0.f, mxp = 0.f;
  // step St of the max chain over the tile's 16 SB scores, CH steps: value f of the chain is
  // register f / SB of block f % SB
  constexpr int CH = 8 * C::SB;
  auto max_step = [&](auto St) {
    constexpr int st = decltype(St)::value;
    if constexpr (C::SB == 2) {
      if constexpr (st == 0) mxp = max3f(s0[0], s0[1], s1[0]);
      else if constexpr (st == 1) mxp = max3f(mxp, s1[1], s0[2]);
      else if constexpr (st < 15) mxp = max3f(mxp, s1[st], s0[st + 1]);
      else mxp = max3f(mxp, s1[15], s1[15]);
    } else {
      constexpr int NV = 16 * C::SB;
      auto v = [&](auto F) -> float { constexpr int f = decltype(F)::value; return sacc[f % C::SB][f / C::SB]; };
      if constexpr (st == 0) {
        mxp = max3f(v(std::integral_constant<int, 0>{}), v(std::integral_constant<int, 1>{}),
                    v(std::integral_constant<int, 2>{}));
      } else {
        constexpr int f1 = 2 * st + 1, f2 = (2 * st + 2 < NV) ? 2 * st + 2 : NV - 1;
        mxp = max3f(mxp, v(std::integral_constant<int, f1>{}), v(std::integral_constant<int, f2>{}));
      }
    }
  };
  auto max_halves = [&](float x) {  // across the two lane halves, without fmaxf's canonicalising
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto row_max_now = [&]() {
    static_for<CH>([&](auto St) { max_step(St); });
    smax_pre = max_halves(mxp);
  };
  auto fence_acc = [&]() {
    if constexpr (C::SB == 2)
      asm volatile("" : "+v"(s0), "+v"(s1));
    else
      asm volatile("" : "+v"(sacc[0]), "+v"(sacc[1]), "+v"(sacc[2]), "+v"(sacc[3]));
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb) asm volatile("" : "+v"(oacc[mb]));
  };
  // MFMA phase j: S_j and O += P_{j-1} V_{j-1} as an explicit pipeline (see fa_fwd.hip).
  auto mfma_phase = [&](auto load_tag, int j, const char* kbuf, const char* vbuf, char* kdst, char* vdst) {
    constexpr int NS = C::SB * C::KSTEPS, NP = C::PH * C::DBLK, N = NS + NP, L = FA8_LOOKAHEAD;
    constexpr int NDMA = decltype(load_tag)::value ? 2 * C::DMA_PER_WAVE : 0;
    constexpr int DMA_EVERY = N / (NDMA > 0 ? NDMA : 1);
    const FA_LDS char* kt = (const FA_LDS char*)kbuf;
    const FA_LDS char* vt = (const FA_LDS char*)vbuf;
    i32x8_t frag[L + 1];
    auto read = [&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < NS)
        frag[i % (L + 1)] = kfrag(kt, i % C::SB, i / C::SB);
      else
        frag[i % (L + 1)] = vfrag(vt + ((i - NS) / C::DBLK) * 64 * C::RB, (i - NS) % C::DBLK);
    };
#if FA_DEBUG_POISON_LDS
    if constexpr (NDMA > 0) {  // the slots K_(j+1) and V_j are loaded into are retired
#pragma unroll
      for (int d = 0; d < C::DMA_PER_WAVE; ++d) {
        poison16((FA_LDS char*)(kdst + (lw * C::DMA_PER_WAVE + d) * 1024 + lane * 16), kPoisonE4M3);
        poison16((FA_LDS char*)(vdst + (lw * C::DMA_PER_WAVE + d) * 1024 + lane * 16), kPoisonE4M3);
      }
      poison_done();
    }
#endif
    if constexpr (CAUSAL && FA_CAUSAL_SKIP) {
      if (j >= j_last + 2) {  // tiles j - 1 and j lie wholly past this wave's diagonal: loads only
        static_for<NDMA>([&](auto I) {
          constexpr int d = decltype(I)::value;
          if constexpr (d < C::DMA_PER_WAVE)
            issue_one(Kh, j + 1, kdst, d);
          else
            issue_one(Vh, j, vdst, d - C::DMA_PER_WAVE);
        });
        return;
      }
    }
#pragma unroll
    for (int b = 0; b < C::SB; ++b) sacc[b] = f32x16_t{};
    static_for<L>([&](auto I) { read(I); });
    static_for<N>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < NS) {
        sacc[i % C::SB] = mfma8(frag[i % (L + 1)], qf[i / C::SB], sacc[i % C::SB]);
      } else {
        constexpr int h = (i - NS) / C::DBLK, mb = (i - NS) % C::DBLK;
        oacc[mb] = mfma8(frag[i % (L + 1)], pb[h], oacc[mb]);
      }
      if constexpr (i + L < N) read(std::integral_constant<int, i + L>{});
      // the max chain over this phase's S, from the second P V slot on (S is complete by then)
      constexpr int SPS = (CH + (NP - 2)) / (NP - 1);  // steps per slot over slots NS + 1 .. N - 1
      if constexpr (i >= NS + 1) {
        constexpr int k0 = (i - NS - 1) * SPS;
        static_for<SPS>([&](auto T) {
          constexpr int st = k0 + decltype(T)::value;
          if constexpr (st < CH) max_step(std::integral_constant<int, st>{});
        });
      }
      if constexpr (i == N - 1) smax_pre = max_halves(mxp);
      if constexpr (NDMA > 0 && i % DMA_EVERY == 0 && i / DMA_EVERY < NDMA) {
        constexpr int d = i / DMA_EVERY;
        if constexpr (d < C::DMA_PER_WAVE)
          issue_one(Kh, j + 1, kdst, d);
        else
          issue_one(Vh, j, vdst, d - C::DMA_PER_WAVE);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    fence_acc();
    asm volatile("" : "+v"(smax_pre));
  };

  // Softmax phase j: mask, lazy max, P_j = exp2(S_j * sl2 - m + kBias) rounded to E4M3, row sums.
  auto softmax_phase = [&](int j) {
    if constexpr (CAUSAL && FA_CAUSAL_SKIP) {
      if (j > j_last) return;  // every score of the tile is masked for this wave: P = 0
    }
    const int tile0 = tile_of(j) * C::BC;
    if ((tile0 + C::BC > Nk) || (CAUSAL && tile0 + C::BC - 1 > q_wave0 + diag)) {
      const int lim = CAUSAL ? min(Nk - 1, q_wave0 + l32 + diag) : Nk - 1;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int key = tile0 + 8 * (jj >> 2) + 4 * hh + (jj & 3);
#pragma unroll
        for (int b = 0; b < C::SB; ++b)
          if (key + 32 * b > lim) sacc[b][jj] = -INFINITY;
      }
      row_max_now();
    }
    const float mx = smax_pre * sl2;
    if (__builtin_amdgcn_ballot_w64(mx > m2 + kTau) != 0) {
      const float mnew = fmaxf(m2, mx);
      const float alpha = fast_exp2(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < C::DBLK; ++mb) oacc[mb] *= alpha;
    }
    const float nm = kBias - m2;
    float rs;
#pragma unroll
    for (int hw = 0; hw < 8 * C::PH; ++hw) {
      const int h = hw >> 3, w = hw & 7;
      const f32x16_t& s = sacc[2 * h + (w >= 4 ? 1 : 0)];
      const int j0 = 4 * (w & 3);
      const float p0 = fast_exp2(__builtin_fmaf(s[j0], sl2, nm));
      const float p1 = fast_exp2(__builtin_fmaf(s[j0 + 1], sl2, nm));
      const float p2 = fast_exp2(__builtin_fmaf(s[j0 + 2], sl2, nm));
      const float p3 = fast_exp2(__builtin_fmaf(s[j0 + 3], sl2, nm));
      rs = hw == 0 ? (p0 + p1) + (p2 + p3) : rs + ((p0 + p1) + (p2 + p3));
      // the low half is written here and the high half by the next conversion, so the word's old
      // contents (the previous tile's codes, already in the register) need no clearing
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pb[h][w], false);
      pb[h][w] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
    }
    lsum += rs;
    if constexpr (C::PH == 1)
      asm volatile("" : "+v"(pb[0]), "+v"(lsum), "+v"(m2));
    else
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(lsum), "+v"(m2));
  };

  auto bar = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
  constexpr std::integral_constant<bool, true> LOAD{};
  constexpr std::integral_constant<bool, false> NOLOAD{};

  if (group == 0) issue(Kh, 0, kb0);
  wait_loads();
  bar();
  if (group == 0) {
    issue(Kh, 1, kb1);
    issue(Vh, 0, vb0);
    qk(kb0);
    fence_acc();
    row_max_now();
    bar();
    int j = 1;
    for (; j + 1 < n; j += 2) {
      softmax_phase(j - 1);
      wait_loads();
      bar();
      mfma_phase(LOAD, j, kb1, vb0, kb0, vb1);
      bar();
      softmax_phase(j);
      wait_loads();
      bar();
      mfma_phase(LOAD, j + 1, kb0, vb1, kb1, vb0);
      bar();
    }
    if (j < n) {
      softmax_phase(j - 1);
      wait_loads();
      bar();
      mfma_phase(LOAD, j, kb1, vb0, kb0, vb1);
      bar();
      ++j;
    }
    softmax_phase(n - 1);
    wait_loads();
    bar();
    if (!(CAUSAL && FA_CAUSAL_SKIP) || n - 1 <= j_last) pv(((n - 1) & 1) ? vb1 : vb0);
    bar();
    bar();
  } else {
    bar();
    qk(kb0);
    fence_acc();
    row_max_now();
    bar();
    int j = 1;
    for (; j + 1 < n; j += 2) {
      softmax_phase(j - 1);
      bar();
      mfma_phase(NOLOAD, j, kb1, vb0, kb0, vb1);
      bar();
      softmax_phase(j);
      bar();
      mfma_phase(NOLOAD, j + 1, kb0, vb1, kb1, vb0);
      bar();
    }
    if (j < n) {
      softmax_phase(j - 1);
      bar();
      mfma_phase(NOLOAD, j, kb1, vb0, kb0, vb1);
      bar();
      ++j;
    }
    softmax_phase(n - 1);
    bar();
    if (!(CAUSAL && FA_CAUSAL_SKIP) || n - 1 <= j_last) pv(((n - 1) & 1) ? vb1 : vb0);
    bar();
  }

  // ---- epilogue: O = v_scale * O_acc / l (RNE to bf16), LSE = (m - kBias + log2 l) * ln 2
  uint16_t* Oh = O + (int64_t)bh * Nq * D;
  float* Lh = LSE + (int64_t)bh * Nq;
  const float l = sum_across_halves(lsum);
  const float inv = vsc / l;
  const int q = q_wave0 + l32;
  // The wave's 32 output rows are one contiguous 32 x D bf16 block: transposed through the wave's
  // LDS staging area (16-byte chunks XOR-swizzled by the row), then stored as whole rows.  The
  // lane index sits behind an empty asm so that the staging addresses are not hoisted into the
  // tile loop.
  constexpr int ORB = D * 2, OCPR = ORB / 16;  // output bytes and 16-byte chunks per row
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int r32 = ln & 31, h2 = ln >> 5;
  FA_LDS char* st = (FA_LDS char*)(stg + wave * 32 * ORB);
#pragma unroll
  for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      u32x2_t w;
      w[0] = pack_bf16x2(oacc[mb][4 * jg + 0] * inv, oacc[mb][4 * jg + 1] * inv);
      w[1] = pack_bf16x2(oacc[mb][4 * jg + 2] * inv, oacc[mb][4 * jg + 3] * inv);
      const int chunk = 4 * mb + jg;
      *(FA_LDS u32x2_t*)(st + r32 * ORB + ((chunk ^ (r32 % OCPR)) << 4) + 8 * h2) = w;
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 32 * ORB / 1024; ++i) {
    const int flat = i * 1024 + ln * 16;
    const int row = flat / ORB, chunk = (flat % ORB) >> 4;
    const u32x4_t v = lds_load16(st + row * ORB + ((chunk ^ (row % OCPR)) << 4));
    if (q_wave0 + row < Nq) *(u32x4_t*)(Oh + (int64_t)(q_wave0 + row) * D + chunk * 8) = v;
  }
  if (q < Nq && hh == 0) Lh[q] = (m2 - kBias + fast_log2(l)) * kLn2;
}

// Persistent kernel with the work items of fwd_bf16_kernel (paired causal blocks, XCD ranges).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ Qs, const float* __restrict__ Ks, const float* __restrict__ Vs, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int Nq, int Nk, int n_qblk, int n_items, int items_per_head, int xcd_split, float sl2,
    int H, int group, int diag, int paired) {
  using C = Fp8Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char kb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[C::TILE_BYTES];
  // Per-wave staging of the bf16 output block (epilogue only); its smaller alignment places it
  // after the rings, whose LDS offsets then stay within the ds_read immediate range.
  __shared__ __attribute__((aligned(16))) char stg[C::WAVES * 32 * D * 2];

  // Zero-fill the rings once, so that no K/V row a masked score meets ever holds a non-finite value.
  {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = threadIdx.x * 16; i < C::TILE_BYTES; i += C::THREADS * 16) {
      lds_store16((FA_LDS char*)(kb0 + i), z);
      lds_store16((FA_LDS char*)(kb1 + i), z);
      lds_store16((FA_LDS char*)(vb0 + i), z);
      lds_store16((FA_LDS char*)(vb1 + i), z);
    }
    __syncthreads();
  }
  const int g = blockIdx.x;
  int it = g, it_end = n_items, stride = gridDim.x;
  if (xcd_split) {
    const int per = n_items >> 3;
    it = (g & 7) * per + (g >> 3);
    it_end = (g & 7) * per + per;
    stride = gridDim.x >> 3;
  }
  for (; it < it_end; it += stride) {
    const int bh = it / items_per_head, r = it % items_per_head;
    const int kvh = (bh / H) * (H / group) + (bh % H) / group;
    const float sl2h = sl2 * Qs[bh] * Ks[kvh];
    const float vsc = Vs[kvh];
    const int qa = CAUSAL ? n_qblk - 1 - r : r;
    const int cnt = (CAUSAL && paired && r != qa) ? 2 : 1;
    for (int k = 0; k < cnt; ++k)
      fp8_block<D, CAUSAL>(Q, K, V, O, LSE, Nq, Nk, sl2h, vsc, bh, kvh, diag, k == 0 ? qa : r, n_qblk, kb0, kb1, vb0,
                           vb1, stg);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fp8_impl(const FwdFp8Args& a, hipStream_t stream) {
  using C = Fp8Cfg<D>;
  const int n_qblk = (a.Nq + C::BR - 1) / C::BR;
  const int paired = (CAUSAL && (int64_t)a.B * a.H * ((n_qblk + 1) / 2) >= a.num_cus) ? 1 : 0;
  const int items_per_head = paired ? (n_qblk + 1) / 2 : n_qblk;
  const int64_t n_items = (int64_t)a.B * a.H * items_per_head;
  const int64_t grid = n_items < a.num_cus ? n_items : a.num_cus;
  const int xcd_split = (grid % 8 == 0 && n_items % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.q_scale, a.k_scale, a.v_scale,
                     (uint16_t*)a.o, a.lse, a.Nq, a.Nk, n_qblk, (int)n_items, items_per_head, xcd_split,
                     a.scale * kLog2e, a.H, a.H / a.H_kv, a.diag, paired);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdFp8Args& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_fp8_impl<128, true>(a, stream) : launch_fp8_impl<128, false>(a, stream);
  return a.causal ? launch_fp8_impl<64, true>(a, stream) : launch_fp8_impl<64, false>(a, stream);
}

}  // namespace fa
