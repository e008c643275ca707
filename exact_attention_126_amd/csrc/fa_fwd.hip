// Fused attention forward for gfx950: O = softmax(scale * Q K^T) V and LSE per row, in one
// kernel.  Method (Day-21 page "GPU 学习日报 Day 21：FlashAttention：GPU Memory Hierarchy 下的 IO
// 优化", §4 tiling and §5.2-5.3 online softmax; Q31 answer "FlashAttention 为什么快", §2):
// each workgroup owns a block of query rows and streams every K/V tile once through LDS; per
// row it keeps a running max m, a running sum l and a rescaled output accumulator, so the
// N x N score and probability matrices never exist outside registers.  One workgroup per
// (batch, head, query block) is the sequence-length parallelism of the Day-21 page §6.
//
// gfx950 mapping (bf16 path):
//  * Transposed products.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K tile from LDS,
//    B = Q^T held in VGPRs for the whole query block) puts one query per lane column: lane l holds
//    query l % 32 and 16 of the 32 keys of an MFMA block, the other 16 sit in lane l ^ 32.
//    Row max and row sum are then in-lane reductions plus one permlane32 swap, and the
//    rescale factor exp2(m_old - m_new) is a per-lane scalar.
//  * O^T = V^T P^T on the same MFMA: the S^T accumulator, converted to bf16, is directly the
//    B operand (P^T).  To make that true, the K row each A-operand lane reads is permuted
//    (key_of_row below) so that the 8 accumulator values lane-half h feeds to k-step t are
//    keys 16t + 8h + 0..7 in order.
//  * V stays in its natural [key][dim] layout in LDS and is read with the transposing
//    ds_read_b64_tr_b16, two reads giving the 8 consecutive keys of one dim an A-operand
//    lane needs.
//  * LDS rows are XOR-swizzled in 16-byte chunks by the row's low four bits, chosen so that
//    the tile stores, the K operand reads and the transposing V reads are all free of bank
//    conflicts.
//  * Ping-pong.  A workgroup is eight waves in two groups of four; each SIMD runs one wave of
//    each group (at most 256 VGPRs per lane, one workgroup per CU).  Workgroup barriers cut
//    time into half-periods; in each, one group issues the MFMAs of S_j and of O += P_{j-1}
//    V_{j-1} while the other runs the softmax of its tile on the VALU, and the groups swap.
//    Empty asm statements that take the phase's results as operands keep the compiler from
//    moving one phase's arithmetic into the next.
//  * K/V tiles live in two-slot LDS rings and are fetched with buffer_load_dwordx4 ... lds, which
//    writes HBM/L2 data straight into LDS without passing through VGPRs; the loads are issued
//    by group 0 inside its MFMA phases and have two half-periods to land.  The buffer form (not
//    global_load_lds) matters: the compiler counts only the buffer form's completion on the
//    vector-memory counter, so its waits for the phase's outstanding LDS reads stay partial
//    instead of draining every read in flight at each load.
//  * The running max is raised lazily: the O_acc rescale is skipped unless some row's max grew
//    by more than 2^8 (the exponentials stay below 256; the result does not depend on the
//    subtracted value).  The bf16 rounding of each tile's largest exponential is carried in a
//    second sum that joins the normaliser of O only, so a key that dominates its row is not
//    left with that rounding (LSE uses the fp32 sum alone).
//  * Causal: every wave processes all the tiles its workgroup needs and masks, element by
//    element, the tiles that reach past its own diagonal (a tile wholly past it contributes
//    nothing); uniform work keeps the two groups in lockstep.  Query blocks with the most
//    tiles are dispatched first, and workgroups are remapped so that the ones an XCD runs
//    together share a head's K/V in that XCD's L2.
//  * The output leaves through LDS: each wave's 32 x D output block is contiguous in HBM, so it is
//    transposed in a per-wave staging area and written with 16-byte stores covering whole rows
//    (stored straight from the accumulator layout, every store instruction touched 32 rows and
//    the next block's first wait sat behind them).
//  * exp is the hardware exp2 with scale * log2(e) folded into one FMA; LSE is emitted in
//    natural-log units.
#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile_layout.h"

namespace fa {
namespace {

template <int D, int BCK = 64>
struct Bf16Cfg {
  static constexpr int WAVES = 8;        // two groups of four, one wave of each per SIMD
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BR = WAVES * 32;  // query rows per workgroup, 32 per wave
  static constexpr int BC = BCK;         // keys per tile
  static constexpr int SB = BC / 32;     // 32-key blocks of S^T per tile
  static constexpr int PG = BC / 16;     // 16-key groups of P^T per tile (k-steps of O^T += V^T P^T)
  static constexpr int RB = D * 2;       // bytes per LDS row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * RB;
  static constexpr int ROWS_PER_DMA = 64 / CPR;                     // rows one wave-wide 1 KiB LDS load fills
  static constexpr int LOADERS = 4;                                 // waves of group 0 move the tiles
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / LOADERS;  // per tensor and tile
  static constexpr int KSTEPS = D / 16;                             // MFMA k-steps of S^T = K Q^T
  static constexpr int DBLK = D / 32;                               // 32-dim blocks of O^T
  static_assert(TILE_BYTES % (1024 * LOADERS) == 0, "tile must split evenly into wave loads");
  struct QFrag {
    bf16x8_t f[KSTEPS];
  };
};

// The masked forward's view of its tile classification (mask_classify_kernel): per query block
// the count and the key-ordered list of non-empty 64-key tiles, bit 15 set on a partial one; the
// bit-packed element mask (one 64-bit word per query row and tile); and the LDS copy of the
// current block's list.  Unused (null) without a mask.
struct MaskView {
  const int* counts;
  const uint16_t* lists;
  const uint64_t* words;
  int nT;        // 64-key tiles per row, ceil(Nk / 64)
  uint16_t* tl;  // LDS, kMaxMaskTiles entries
  // Dynamic schedule: items (query block, head) in block-major order with the blocks by falling
  // tile count (order); the next item of the workgroup, claimed before the block by its first
  // thread (LDS word claim), is read after the block's first barrier into *next_item.
  const FA_LDS int* order = nullptr;  // kMaxRankedBlocks entries; blocks past them keep their index
  const FA_LDS int* claim = nullptr;
  int* next_item = nullptr;
  int n_items = 0, nbh_all = 0, H = 0, group = 0;
};

// Lazy rescaling threshold, log2 units: the running max used for the exponentials is only
// raised when a tile's row max exceeds it by more than this, so most tiles skip the
// O_acc rescale.  Exponentials are then bounded by 2^kLazyRescale (exact: softmax does not
// depend on the value subtracted, Day-21 page §5.2).
constexpr float kLazyRescale = 8.f;

// Query blocks the masked forward ranks by tile count for its schedule (two LDS arrays of ints).
constexpr int kMaxRankedBlocks = 2048;

#ifndef FA_D64_TILE
#define FA_D64_TILE 128  // keys per tile of the d = 64 forward without an element mask
#endif
// Keys per tile: 64, and FA_D64_TILE at d = 64 without an element mask (the tile classification of
// the masked forward is per 64 keys).  A larger tile at d = 64 halves the barriers and the per-tile
// work of the softmax (decision, tile loads) per key; at d = 128 its accumulators would not fit.
template <int D, bool MASKED>
constexpr int kTileKeys = (D == 64 && !MASKED) ? FA_D64_TILE : 64;

#ifndef FA_CAUSAL_SKIP
#define FA_CAUSAL_SKIP 1  // causal: a wave skips the products and softmax of tiles past its diagonal
#endif

#ifndef FA_LOOKAHEAD
#define FA_LOOKAHEAD 8  // MFMAs by which LDS operand reads run ahead
#endif

// Q^T fragments (the B operand of S^T = K Q^T) of the 32 queries from qw0 of query head bh:
// lane (l32, hh) holds dims 16 ks + 8 hh .. + 7 of query qw0 + l32 (clamped to the last query).
template <int D>
__device__ __forceinline__ void load_q_frags(bf16x8_t (&qf)[Bf16Cfg<D>::KSTEPS], const uint16_t* __restrict__ Q,
                                             int bh, int Nq, int qw0, int l32, int hh) {
  const int qrow = min(qw0 + l32, Nq - 1);
  const uint16_t* qp = Q + ((int64_t)bh * Nq + qrow) * D + 8 * hh;
#pragma unroll
  for (int ks = 0; ks < Bf16Cfg<D>::KSTEPS; ++ks) qf[ks] = as_bf16x8(gload16(qp + 16 * ks));
}

// Eight waves: group 0 (waves 0-3) and group 1 (waves 4-7) each cover the four SIMDs, so every
// SIMD runs one wave of each group.  Time is cut into half-periods separated by workgroup
// barriers.  In half-period h a wave of group g works on phase p = h - g:
//   p = 2j     MFMA phase j:    S_j = K_j Q^T, then O += P_{j-1} V_{j-1}
//   p = 2j + 1 softmax phase j: max, lazy rescale, P_j = exp2(S_j - m) (VALU)
// so on every SIMD one wave feeds the matrix core while the other runs its softmax.  Loads of
// K_{j+1} and V_j start at half-period 2j and are complete two half-periods later.
// One query block (batch*head bh, rows qblk*BR ..) of the forward, run by the whole workgroup
// with the LDS rings kb0/kb1 (K) and vb0/vb1 (V).  The first barrier it executes orders its LDS
// use after the previous block's; its last barrier is passed only when every wave is done.
template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ bool fwd_block(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                          float* __restrict__ LSE, int Nq, int Nk, float sl2, int bh, int kvh,
                                          int diag, int qblk, int n_qblk, char* kb0, char* kb1, char* vb0,
                                          char* vb1, char* stg, bf16x8_t (&qf)[Bf16Cfg<D>::KSTEPS], bool pre,
                                          bool has_next, int nbh, int nkvh, int nqblk, const MaskView& mk) {
  using C = Bf16Cfg<D, kTileKeys<D, MASKED>>;
  static_assert(!MASKED || C::BC == 64, "the mask classification lists 64-key tiles");
  const uint16_t* Kh = K + (int64_t)kvh * Nk * D;
  const uint16_t* Vh = V + (int64_t)kvh * Nk * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int q_wave0 = qblk * C::BR + wave * 32;  // first query of this wave (wave-uniform)
  // Causal: the last tile with a key this wave's rows can see.  Every key of a later tile lies past
  // the diagonal of all its rows: its scores would all be -inf, its P all 0 and its running max
  // unchanged, so the wave skips the tile's products and softmax (bit for bit the same result)
  // and only keeps its part of the workgroup's barriers and tile loads.  Fewer products and
  // exponentials cost less energy, and the kernel is held by the clock the power limit allows.
  const int j_last = (CAUSAL && FA_CAUSAL_SKIP) ? (q_wave0 + 31 + diag) / C::BC : 0;

  // ---- Q^T fragments (B operand) of this block are already in qf: the previous block (or the
  // kernel, for the first one) loaded them.  This block loads the next block's (its own again when
  // none follows) at the start of its last softmax phase, after its last S product.

  // ---- the workgroup streams n tiles and every wave processes all of them.  Without a mask the
  // tile order is free, so query blocks of one head start at different tiles (rotation rot):
  // the workgroups working on a head then stream different parts of its K/V at any moment
  // instead of all asking the L2 for the same lines.  Step t visits tile (t + rot) mod n; the
  // extra step t = n (a dummy reload of the free slot) maps to a valid tile too.
  // With a mask the block walks its list of non-empty tiles in key order instead (copied to LDS
  // here, read after the block's first barrier); its first entry is read from global memory for
  // the load issued before that barrier.  Tile indices are wave-uniform and kept in scalars.
  int n, rot = 0, first_tile = 0;
  if constexpr (MASKED) {
    const uint16_t* lst = mk.lists + (int64_t)qblk * mk.nT;
    n = __builtin_amdgcn_readfirstlane(mk.counts[qblk]);
    if (n > 0) first_tile = __builtin_amdgcn_readfirstlane((int)(lst[0] & 0x7FFF));
    for (int i = tid; i < n; i += C::THREADS) mk.tl[i] = lst[i];
  } else {
    const int kv_end = CAUSAL ? min(Nk, qblk * C::BR + C::BR + diag) : Nk;
    n = (kv_end + C::BC - 1) / C::BC;
    rot = CAUSAL ? 0 : (int)(((int64_t)qblk * n) / n_qblk);
  }
  auto tile_of = [&](int t) {
    if constexpr (MASKED) {
      return (t == 0 || t >= n) ? first_tile : __builtin_amdgcn_readfirstlane((int)(mk.tl[t] & 0x7FFF));
    } else {
      const int x = t + rot;
      return x >= n ? x - n : x;
    }
  };
  // a partial tile of the mask: some of its keys are visible to some rows of the block
  auto partial = [&](int t) { return MASKED && __builtin_amdgcn_readfirstlane((int)mk.tl[t]) >= 0x8000; };

  // With a mask: the workgroup's next item, published by the barrier before this call site; its
  // head and query block replace the next-block arguments (used for the Q prefetch).
  auto take_claim = [&]() {
    if constexpr (MASKED) {
      const int nxt = __builtin_amdgcn_readfirstlane(*mk.claim);
      *mk.next_item = nxt;
      has_next = nxt < mk.n_items;
      if (has_next) {
        nbh = nxt % mk.nbh_all;
        const int k = nxt / mk.nbh_all;
        nqblk = k < kMaxRankedBlocks ? __builtin_amdgcn_readfirstlane(mk.order[k]) : k;
        nkvh = (nbh / mk.H) * (mk.H / mk.group) + (nbh % mk.H) / mk.group;
      }
    }
  };
  if constexpr (MASKED) {
    if (n == 0) {
      // No row of the block sees any key: O = 0 and LSE = ln 0 = -inf.  The next block's Q
      // fragments are loaded here, as a block with tiles would in its last phase, once the
      // workgroup's claim of its next item is visible to every wave.
      __syncthreads();
      take_claim();
      load_q_frags<D>(qf, Q, nbh, Nq, nqblk * C::BR + wave * 32, l32, hh);
      uint16_t* Oh = O + (int64_t)bh * Nq * D;
      const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 32 * C::RB / 1024; ++i) {
        const int flat = i * 1024 + lane * 16;
        const int row = flat / C::RB, chunk = (flat % C::RB) >> 4;
        if (q_wave0 + row < Nq) *(u32x4_t*)(Oh + (int64_t)(q_wave0 + row) * D + chunk * 8) = z;
      }
      if (q_wave0 + l32 < Nq && hh == 0) LSE[(int64_t)bh * Nq + q_wave0 + l32] = -INFINITY;
      return false;
    }
  }

  // ---- asynchronous global -> LDS tile loads, issued by the four waves of group 0 inside their
  // MFMA phases (their vector units are idle there).  One instruction moves 16 bytes per lane
  // into 1 KiB of consecutive LDS; lane L lands in row L / CPR, slot L % CPR of its rows, so it
  // fetches the global chunk that the row's swizzle puts in that slot.  Each tile gets its own
  // buffer resource, starting at the tile's first key and ending at the last key of the head, so
  // the per-lane byte offset is the same for every tile and a load costs no vector instruction.
  // Rows past the last key fall outside the resource: the hardware range check returns zeros
  // for them without touching memory (their scores are masked; the LDS rings are zero-filled at
  // kernel start, so those rows hold finite values in any case).
  const int lw = wave & 3;
  int dma_off[C::DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
    const int row = (lw * C::DMA_PER_WAVE + i) * C::ROWS_PER_DMA + lane / C::CPR;
    dma_off[i] = row * C::RB + ((lane % C::CPR) ^ swz<D>(row)) * 16;
  }
  // With an even tile count the step past the last tile reloads into kb0; when a next block
  // follows, that load fetches the next block's first K tile instead (it lands in kb0, where the
  // next block expects it), and the next block skips its own first load, wait and barrier.
  const bool do_pf = !MASKED && has_next && (n % 2 == 0);
  const uint16_t* nKh = K + (int64_t)nkvh * Nk * D;
  const int nrot = CAUSAL ? 0 : (int)(((int64_t)nqblk * n) / n_qblk);
  auto issue_one = [&](const uint16_t* src, int t, char* buf, int i) {
    const bool nxt = do_pf && t >= n;
    const int r0 = (nxt ? nrot : tile_of(t)) * C::BC;
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc((nxt ? nKh : src) + (int64_t)r0 * D, (Nk - r0) * C::RB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(buf + (lw * C::DMA_PER_WAVE + i) * 1024), 16, dma_off[i], 0, 0, 0);
  };
  auto issue = [&](const uint16_t* src, int t, char* buf) {
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) issue_one(src, t, buf, i);
  };

  // ---- per-lane LDS read offsets
  int koff[C::KSTEPS];
  {
    const int krow = key_of_row(l32);
    const int ks_sw = swz<D>(krow);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) koff[ks] = krow * C::RB + (((2 * ks + hh) ^ ks_sw) << 4);
  }
  int voff[C::DBLK][2];
  {
    const int g = lane >> 4, s = lane & 15;
    const int vh = g >> 1, ve = s >> 2, vq = s & 3;
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const int key = 8 * vh + 4 * I + ve;
        const int dim = 32 * mb + 16 * (g & 1) + 4 * vq;
        voff[mb][I] = key * C::RB + (((dim >> 3) ^ swz<D>(key)) << 4) + ((dim >> 2) & 1) * 8;
      }
  }

  f32x16_t oacc[C::DBLK];
#pragma unroll
  for (int mb = 0; mb < C::DBLK; ++mb) oacc[mb] = f32x16_t{};
  // m2: running max used for the exponentials (log2 units); lsum: this lane half's share of the
  // row sum of the fp32 exponentials (for l and LSE); csum: the bf16 rounding error of each tile's
  // largest exponential, summed (the same in both lane halves; it joins l only where O is
  // normalised, see softmax_phase).
  float m2 = -INFINITY, lsum = 0.f, csum = 0.f;
  f32x16_t sacc[C::SB];  // S^T of the current tile, 32-key blocks
  f32x16_t& s0 = sacc[0];
  f32x16_t& s1 = sacc[1];
  // With a mask: the lane's row's 64-bit mask word for the tile whose softmax comes next, loaded
  // one softmax phase ahead (the one for the first tile before the loop).
  const uint64_t* mrow = nullptr;
  uint64_t mword = 0;
  if constexpr (MASKED) {
    mrow = mk.words + (int64_t)min(q_wave0 + l32, Nq - 1) * mk.nT;
    mword = mrow[first_tile];
  }
  u32x4_t pb[C::PG];  // bf16 P^T of the previous tile, 16-key groups

  // S_j = K_j Q^T
  auto qk = [&](const char* kbuf) {
    const FA_LDS char* kt = (const FA_LDS char*)kbuf;
#pragma unroll
    for (int b = 0; b < C::SB; ++b) sacc[b] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      bf16x8_t a[C::SB];
#pragma unroll
      for (int b = 0; b < C::SB; ++b) a[b] = as_bf16x8(lds_load16(kt + b * 32 * C::RB + koff[ks]));
#pragma unroll
      for (int b = 0; b < C::SB; ++b) sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[b], qf[ks], sacc[b], 0, 0, 0);
    }
  };
  // O^T += V^T P^T of the previous tile
  auto pv = [&](const char* vbuf) {
    const FA_LDS char* vt = (const FA_LDS char*)vbuf;
#pragma unroll
    for (int t = 0; t < C::PG; ++t)
#pragma unroll
      for (int mb = 0; mb < C::DBLK; ++mb) {
        const i16x4_t lo = lds_load8_tr16(vt + voff[mb][0] + t * 16 * C::RB);
        const i16x4_t hi = lds_load8_tr16(vt + voff[mb][1] + t * 16 * C::RB);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pb[t]), oacc[mb], 0, 0, 0);
      }
  };
  // At D = 64 (EARLY_MAX) the tile's largest raw score of this lane's row, for tiles that need no
  // element mask, is taken in the MFMA phase that computes S, under its P V products: its sixteen
  // dependent max3 steps and the swap across the lane halves.  One wave issues a VALU instruction
  // only every few cycles, and at D = 64 the softmax phase is twice as long as the MFMA phase, so
  // moving the steps shortens every half-period (+3%).  At D = 128 the two phases are nearly equal
  // and the extra VALU work beside the MFMAs costs more than it saves (-0.5 to -1.7%, measured):
  // the max stays in the softmax phase.
  constexpr bool EARLY_MAX = (D == 64);
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
  // Pins the MFMA results to the phase that computes them (see the fence in softmax_phase).
  auto fence_acc = [&]() {
    if constexpr (C::SB == 2)
      asm volatile("" : "+v"(s0), "+v"(s1));
    else
      asm volatile("" : "+v"(sacc[0]), "+v"(sacc[1]), "+v"(sacc[2]), "+v"(sacc[3]));
#pragma unroll
    for (int mb = 0; mb < C::DBLK; ++mb) asm volatile("" : "+v"(oacc[mb]));
  };
  // MFMA phase j (0 < j < n): S_j and O += P_{j-1} V_{j-1}, written as an explicit pipeline of
  // NS + NP slots.  Slot i issues MFMA i (S MFMAs first, then the PV MFMAs), then the LDS reads of
  // the A operand of MFMA i + L into a rotating set of L + 1 fragment registers, and, when this
  // wave moves tiles, every DMA_EVERY-th slot one of its global -> LDS loads of K_{j+1} (a
  // harmless reload of a valid tile when j + 1 = n) and V_j into the free slots kdst and vdst.  Scheduling
  // barriers between slots keep the compiler from collapsing the read-ahead.
  auto mfma_phase = [&](auto load_tag, int j, const char* kbuf, const char* vbuf, char* kdst, char* vdst) {
    constexpr int NS = C::SB * C::KSTEPS, NP = C::PG * C::DBLK, N = NS + NP, L = FA_LOOKAHEAD;
    constexpr int NDMA = decltype(load_tag)::value ? 2 * C::DMA_PER_WAVE : 0;
    constexpr int DMA_EVERY = N / (NDMA > 0 ? NDMA : 1);
    const FA_LDS char* kt = (const FA_LDS char*)kbuf;
    const FA_LDS char* vt = (const FA_LDS char*)vbuf;
    bf16x8_t frag[L + 1];
    auto read = [&](auto I) {  // A operand of MFMA I
      constexpr int i = decltype(I)::value;
      if constexpr (i < NS) {
        frag[i % (L + 1)] = as_bf16x8(lds_load16(kt + (i % C::SB) * 32 * C::RB + koff[i / C::SB]));
      } else {
        constexpr int t = (i - NS) / C::DBLK, mb = (i - NS) % C::DBLK;
        const i16x4_t lo = lds_load8_tr16(vt + voff[mb][0] + t * 16 * C::RB);
        const i16x4_t hi = lds_load8_tr16(vt + voff[mb][1] + t * 16 * C::RB);
        frag[i % (L + 1)] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
#if FA_DEBUG_POISON_LDS
    if constexpr (NDMA > 0) {  // the slots K_(j+1) and V_j are loaded into are retired
#pragma unroll
      for (int d = 0; d < C::DMA_PER_WAVE; ++d) {
        poison16((FA_LDS char*)(kdst + (lw * C::DMA_PER_WAVE + d) * 1024 + lane * 16), kPoisonBf16);
        poison16((FA_LDS char*)(vdst + (lw * C::DMA_PER_WAVE + d) * 1024 + lane * 16), kPoisonBf16);
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
        sacc[i % C::SB] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[i % (L + 1)], qf[i / C::SB], sacc[i % C::SB], 0, 0, 0);
      } else {
        constexpr int t = (i - NS) / C::DBLK, mb = (i - NS) % C::DBLK;
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[i % (L + 1)], as_bf16x8(pb[t]), oacc[mb], 0, 0, 0);
      }
      if constexpr (i + L < N) read(std::integral_constant<int, i + L>{});
      // the max chain over this phase's S, from the second P V slot on (S is complete by then)
      constexpr int SPS = (CH + (NP - 3)) / (NP - 2);  // steps per slot over slots NS + 1 .. N - 2
      if constexpr (EARLY_MAX && i >= NS + 1 && i <= N - 2) {
        constexpr int k0 = (i - NS - 1) * SPS;
        static_for<SPS>([&](auto T) {
          constexpr int st = k0 + decltype(T)::value;
          if constexpr (st < CH) max_step(std::integral_constant<int, st>{});
        });
      }
      if constexpr (EARLY_MAX && i == N - 1) smax_pre = max_halves(mxp);
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
    if constexpr (EARLY_MAX) asm volatile("" : "+v"(smax_pre));
  };

  // Softmax phase j: element mask where the tile reaches past the wave's diagonal or the end of
  // the keys (a tile past the diagonal is masked whole and contributes nothing), running max
  // raised lazily with the O_acc rescale, P_j = exp2(S_j * scale * log2 e - m) packed to bf16,
  // row sums into l.
  // With the lazy max the tile's largest exponential lies anywhere in (0, 2^8] instead of being
  // exactly 1, so its bf16 rounding (relative error up to 2^-8) would stay in O: on a row that one
  // key dominates, O = bf16(p) v / p misses v by up to 2^-8 |v|.  That error of the tile's largest
  // exponential, bf16(p_max) - p_max, is added to csum, and O is divided by l + csum: the dominant
  // key's rounding then cancels between O_acc and its normaliser, as if the running max were
  // exact.  LSE keeps the fp32 sum l.
  auto softmax_phase = [&](int j) {
    if constexpr (CAUSAL && FA_CAUSAL_SKIP) {
      if (j > j_last) return;  // every score of the tile is masked for this wave: P = 0
    }
    const int tile0 = tile_of(j) * C::BC;
    uint64_t mcur = 0;
    const bool cut = (tile0 + C::BC > Nk) || (CAUSAL && tile0 + C::BC - 1 > q_wave0 + diag);
    bool edge = cut;
    if constexpr (MASKED) {
      mcur = mword;
      mword = mrow[tile_of(j + 1)];  // the next tile's word (a valid tile's when j + 1 == n)
      edge = edge || partial(j);
    }
    if (edge) {
      if constexpr (MASKED) {
        if (partial(j)) {
          // key 16 (jj / 8) + 8 hh + jj % 8 of the tile is in s0[jj], that key + 32 in s1[jj]
          const uint32_t lo = (uint32_t)(mcur >> (8 * hh)), hi = (uint32_t)(mcur >> (32 + 8 * hh));
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int b = 16 * (jj >> 3) + (jj & 7);
            if (!((lo >> b) & 1u)) s0[jj] = -INFINITY;
            if (!((hi >> b) & 1u)) s1[jj] = -INFINITY;
          }
        }
      }
      if (cut) {
        const int lim = CAUSAL ? min(Nk - 1, q_wave0 + l32 + diag) : Nk - 1;  // last key this lane's query sees
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int key = tile0 + 16 * (jj >> 3) + 8 * hh + (jj & 7);
#pragma unroll
          for (int b = 0; b < C::SB; ++b)
            if (key + 32 * b > lim) sacc[b][jj] = -INFINITY;
        }
      }
    }
    // the row's largest score in this tile, unscaled (already taken in the MFMA phase when
    // EARLY_MAX and no element was masked)
    if (!EARLY_MAX || edge) row_max_now();
    const float smax = smax_pre;
    float mx = smax * sl2;
    if (__builtin_amdgcn_ballot_w64(mx > m2 + kLazyRescale) != 0) {
      const float mnew = fmaxf(m2, mx);
      // with a mask a row may still have seen no key (m2 = mnew = -inf): its sums stay 0
      const float alpha = (MASKED && mnew == -INFINITY) ? 1.f : fast_exp2(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
      csum *= alpha;
#pragma unroll
      for (int mb = 0; mb < C::DBLK; ++mb) oacc[mb] *= alpha;
    }
    // a row that has seen no key yet (mask only) has only -inf scores here: exp2(-inf + 0) = 0
    const float nm = (MASKED && m2 == -INFINITY) ? 0.f : -m2;
    {  // the same FMA and exp2 as that key's own exponential below, so the two round alike
      const float pmax = fast_exp2(__builtin_fmaf(smax, sl2, nm));
      csum += bf16_round(pmax) - pmax;
    }
    float rs;
#pragma unroll
    for (int t = 0; t < C::PG; ++t) {
      const f32x16_t& s = sacc[t >> 1];
      const int j0 = 8 * (t & 1);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float pa = fast_exp2(__builtin_fmaf(s[j0 + 2 * u], sl2, nm));
        const float pc = fast_exp2(__builtin_fmaf(s[j0 + 2 * u + 1], sl2, nm));
        rs = (t == 0 && u == 0) ? pa + pc : rs + (pa + pc);
        pb[t][u] = pack_bf16x2(pa, pc);
      }
    }
    lsum += rs;
    // Keep this phase's vector work in this phase: without the fence the compiler sinks the
    // exponentials past the barrier, next to their use in the other group's MFMA phase.
    if constexpr (C::PG == 4) {
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]), "+v"(lsum), "+v"(m2), "+v"(csum));
    } else {
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]), "+v"(lsum), "+v"(m2), "+v"(csum));
      asm volatile("" : "+v"(pb[4]), "+v"(pb[5]), "+v"(pb[6]), "+v"(pb[7]));
    }
    (void)mcur;
  };

  // Workgroup barrier between half-periods.  It waits for this wave's LDS reads (the slot may
  // be refilled next) but not for its tile loads in flight; those are waited for where due.
  auto bar = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
  // vmcnt(KSTEPS): every tile load is done; the next block's Q loads, issued after them, may not be
  static_assert(C::KSTEPS < 16, "vmcnt field");
  auto wait_loads_but_q = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70 | C::KSTEPS); };
  constexpr std::integral_constant<bool, true> LOAD{};
  constexpr std::integral_constant<bool, false> NOLOAD{};

  if (!pre) {
    if (group == 0) issue(Kh, 0, kb0);
    wait_loads();
    bar();
  }
  if constexpr (MASKED) take_claim();  // a masked block never has its first tile preloaded
  // Slots by tile parity: K_j in kb[j & 1], V_j in vb[j & 1].  Every wave runs 2n + 3 barriers
  // (2n + 2 when the previous block preloaded K_0).
  if (group == 0) {
    issue(Kh, 1, kb1);  // h = 0 (K_1 is a harmless reload of K_0 when n = 1)
    issue(Vh, 0, vb0);
    qk(kb0);
    fence_acc();
    if constexpr (EARLY_MAX) row_max_now();
    bar();
    int j = 1;
    for (; j + 1 < n; j += 2) {
      softmax_phase(j - 1);  // h = 2j - 1
      wait_loads();
      bar();
      mfma_phase(LOAD, j, kb1, vb0, kb0, vb1);  // h = 2j
      bar();
      softmax_phase(j);  // h = 2j + 1
      wait_loads();
      bar();
      mfma_phase(LOAD, j + 1, kb0, vb1, kb1, vb0);  // h = 2j + 2
      bar();
    }
    if (j < n) {  // one more tile (odd j)
      softmax_phase(j - 1);
      wait_loads();
      bar();
      mfma_phase(LOAD, j, kb1, vb0, kb0, vb1);
      bar();
      ++j;
    }
    load_q_frags<D>(qf, Q, nbh, Nq, nqblk * C::BR + wave * 32, l32, hh);
    softmax_phase(n - 1);  // h = 2n - 1
    wait_loads_but_q();
    bar();
    if (!(CAUSAL && FA_CAUSAL_SKIP) || n - 1 <= j_last) pv(((n - 1) & 1) ? vb1 : vb0);  // h = 2n
    bar();
    bar();  // h = 2n + 1: group 1 finishes
  } else {
    bar();  // h = 0: idle
    qk(kb0);  // h = 1
    fence_acc();
    if constexpr (EARLY_MAX) row_max_now();
    bar();
    int j = 1;
    for (; j + 1 < n; j += 2) {
      softmax_phase(j - 1);  // h = 2j
      bar();
      mfma_phase(NOLOAD, j, kb1, vb0, kb0, vb1);  // h = 2j + 1
      bar();
      softmax_phase(j);  // h = 2j + 2
      bar();
      mfma_phase(NOLOAD, j + 1, kb0, vb1, kb1, vb0);  // h = 2j + 3
      bar();
    }
    if (j < n) {
      softmax_phase(j - 1);
      bar();
      mfma_phase(NOLOAD, j, kb1, vb0, kb0, vb1);
      bar();
      ++j;
    }
    load_q_frags<D>(qf, Q, nbh, Nq, nqblk * C::BR + wave * 32, l32, hh);
    softmax_phase(n - 1);  // h = 2n
    bar();
    if (!(CAUSAL && FA_CAUSAL_SKIP) || n - 1 <= j_last) pv(((n - 1) & 1) ? vb1 : vb0);  // h = 2n + 1
    bar();
  }

  // ---- epilogue: O = O_acc / l (RNE to bf16), LSE = (m + log2 l) * ln 2.  The wave's 32 output
  // rows are one contiguous 32 x D block of O; a lane holds 8-byte pieces of one row, so the block
  // is first transposed through the wave's own LDS staging area (16-byte chunks XOR-swizzled by
  // the row) and then written with 16-byte stores that each cover whole rows.
  uint16_t* Oh = O + (int64_t)bh * Nq * D;
  float* Lh = LSE + (int64_t)bh * Nq;
  const float l = sum_across_halves(lsum);
  // a row with no visible key (mask only) has l = 0: O = 0, and LSE = -inf below
  const float inv = (MASKED && !(l + csum > 0.f)) ? 0.f : 1.f / (l + csum);
  const int q = q_wave0 + l32;
  // Lane index behind an empty asm: the staging addresses below are derived from it, so the
  // compiler cannot hoist them into the tile loop, where they would hold registers for nothing.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int r32 = ln & 31, h2 = ln >> 5;
  FA_LDS char* st = (FA_LDS char*)(stg + wave * 32 * C::RB);
#pragma unroll
  for (int mb = 0; mb < C::DBLK; ++mb)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      u32x2_t w;
      w[0] = pack_bf16x2(oacc[mb][4 * jg + 0] * inv, oacc[mb][4 * jg + 1] * inv);
      w[1] = pack_bf16x2(oacc[mb][4 * jg + 2] * inv, oacc[mb][4 * jg + 3] * inv);
      const int chunk = 4 * mb + jg;
      *(FA_LDS u32x2_t*)(st + r32 * C::RB + ((chunk ^ (r32 % C::CPR)) << 4) + 8 * h2) = w;
    }
  // lgkmcnt(0): this wave's staging writes are done; vmcnt(0): the next block's Q fragments have
  // landed (issued two phases ago), so no wait for them lands behind the stores below
  __builtin_amdgcn_s_waitcnt(0x0070);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 32 * C::RB / 1024; ++i) {
    const int flat = i * 1024 + ln * 16;
    const int row = flat / C::RB, chunk = (flat % C::RB) >> 4;
    const u32x4_t v = lds_load16(st + row * C::RB + ((chunk ^ (row % C::CPR)) << 4));
    if (q_wave0 + row < Nq) *(u32x4_t*)(Oh + (int64_t)(q_wave0 + row) * D + chunk * 8) = v;
  }
  if (q < Nq && hh == 0) Lh[q] = (m2 + fast_log2(l)) * kLn2;
  return do_pf;
}

// Persistent kernel: one workgroup per CU loops over work items.  A causal item is the pair of
// query blocks q and n_qblk - 1 - q of one head (heaviest first), so every item streams the
// same number of tiles and the CUs stay balanced; a non-causal item is one query block, and so
// is a causal one when pairing would leave CUs idle (fewer pairs than CUs: the blocks then run
// heaviest first, one per CU, which for a short query chunk against a long cache are nearly
// equal anyway).  With xcd_split, the items of XCD x (workgroups b with b % 8 == x) are a
// contiguous range ordered by head, so the 32 CUs of an XCD work on about two heads at a time and
// share their K/V in that XCD's L2.  The workgroup walks its blocks as one sequence, so each block
// can prefetch the next one's Q fragments and first K tile.  With a mask (MASKED) the items are
// single blocks in order, each walking its own list of non-empty tiles.
template <int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Nq, int Nk, int n_qblk, int n_items, int items_per_head,
    int xcd_split, float sl2, int H, int group, int diag, int paired, const int* __restrict__ mcounts,
    const uint16_t* __restrict__ mlists, const uint64_t* __restrict__ mwords, int nT, int* __restrict__ mqueue) {
  using C = Bf16Cfg<D, kTileKeys<D, MASKED>>;
  static_assert(!(CAUSAL && MASKED), "a causal mask is one element mask among others");
  // LDS copy of the current block's tile list (masked forward only)
  __shared__ uint16_t tl[MASKED ? kMaxMaskTiles : 1];
  const MaskView mk{mcounts, mlists, mwords, nT, tl};
  // Two-slot rings for K and V tiles.  Separate arrays let the compiler see that reads of one
  // slot never alias the asynchronous loads into another.
  __shared__ __attribute__((aligned(1024))) char kb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[C::TILE_BYTES];
  // Per-wave staging of the output block (epilogue only).  Its smaller alignment places it after
  // the rings, whose LDS offsets must stay below 64 KiB to fit the immediate offset of ds_read
  // (placed first, it pushed every ring address past that limit and cost an address add per read).
  __shared__ __attribute__((aligned(16))) char stg[C::WAVES * 32 * C::RB];

  // Zero-fill the rings once, so that no K/V row a masked score meets ever holds a non-finite
  // bit pattern (0 * inf would poison O).
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
  if constexpr (MASKED) {
    // The blocks' tile counts differ (by the mask), so the items (query block, head) are handed out
    // dynamically, heaviest block first: items are block-major over the blocks ranked by falling
    // tile count, workgroup g starts with item g, and before each block its first thread claims the
    // next item from the counter (gridDim.x + the count of earlier claims).  The claim alternates
    // between two LDS words, each read by every wave after the first barrier of the block it was
    // made for.  Every workgroup ranks the blocks itself, in LDS, from the tile counts; past
    // kMaxRankedBlocks blocks they keep their index order (still correct, less balanced).
    __shared__ int s_claim[2];
    __shared__ int s_cnt[kMaxRankedBlocks], s_order[kMaxRankedBlocks];
    const int nbh_all = n_items / n_qblk;
    if (n_qblk <= kMaxRankedBlocks) {
      for (int q = threadIdx.x; q < n_qblk; q += Bf16Cfg<D>::THREADS) s_cnt[q] = mcounts[q];
      __syncthreads();
      for (int q = threadIdx.x; q < n_qblk; q += Bf16Cfg<D>::THREADS) {
        const int c = s_cnt[q];
        int rank = 0;
        for (int p = 0; p < n_qblk; ++p) rank += (s_cnt[p] > c || (s_cnt[p] == c && p < q)) ? 1 : 0;
        s_order[rank] = q;
      }
    } else {
      for (int q = threadIdx.x; q < kMaxRankedBlocks; q += Bf16Cfg<D>::THREADS) s_order[q] = q;
    }
    __syncthreads();
    const FA_LDS int* order = (const FA_LDS int*)s_order;
    auto qblk_at = [&](int k) { return k < kMaxRankedBlocks ? __builtin_amdgcn_readfirstlane(order[k]) : k; };
    int nxt = n_items;
    MaskView md = mk;
    md.order = order;
    md.next_item = &nxt;
    md.n_items = n_items;
    md.nbh_all = nbh_all;
    md.H = H;
    md.group = group;
    typename Bf16Cfg<D>::QFrag qf;
    int item = g, par = 0;
    if (item < n_items) {
      const int qb0 = qblk_at(item / nbh_all);
      load_q_frags<D>(qf.f, Q, item % nbh_all, Nq, qb0 * Bf16Cfg<D>::BR + (threadIdx.x >> 6) * 32, threadIdx.x & 31,
                      (threadIdx.x >> 5) & 1);
    }
    while (item < n_items) {
      const int bh = item % nbh_all;
      const int qblk = qblk_at(item / nbh_all);
      const int kvh = (bh / H) * (H / group) + (bh % H) / group;
      if (threadIdx.x == 0) s_claim[par] = (int)gridDim.x + atomicAdd(mqueue, 1);
      md.claim = (const FA_LDS int*)&s_claim[par];
      fwd_block<D, CAUSAL, MASKED>(Q, K, V, O, LSE, Nq, Nk, sl2, bh, kvh, diag, qblk, n_qblk, kb0, kb1, vb0, vb1, stg,
                                   qf.f, false, false, bh, kvh, qblk, md);
      item = nxt;
      par ^= 1;
    }
    return;
  }
  int it0 = g, it_end = n_items, stride = gridDim.x;
  if (!MASKED && xcd_split) {
    const int per = n_items >> 3;
    it0 = (g & 7) * per + (g >> 3);
    it_end = (g & 7) * per + per;
    stride = gridDim.x >> 3;
  }
  // Item of this workgroup's step r.
  auto item_at = [&](int r) { return it0 + r * stride; };
  // Block k of item it: its head, K/V head and query block, and the number of blocks of the item.
  auto block_of = [&](int item, int k, int& bh, int& kvh, int& qblk) {
    bh = item / items_per_head;
    const int r = item % items_per_head;
    kvh = (bh / H) * (H / group) + (bh % H) / group;  // K/V head of query head bh
    const int qa = CAUSAL ? n_qblk - 1 - r : r;
    qblk = k == 0 ? qa : r;
    return (CAUSAL && paired && r != qa) ? 2 : 1;
  };
  typename Bf16Cfg<D>::QFrag qf;
  bool pre = false;
  int r = 0, k = 0;
  if (item_at(0) < it_end) {
    int bh, kvh, qblk;
    block_of(item_at(0), 0, bh, kvh, qblk);
    load_q_frags<D>(qf.f, Q, bh, Nq, qblk * Bf16Cfg<D>::BR + (threadIdx.x >> 6) * 32, threadIdx.x & 31,
                    (threadIdx.x >> 5) & 1);
  }
  while (item_at(r) < it_end) {
    int bh, kvh, qblk;
    const int cnt = block_of(item_at(r), k, bh, kvh, qblk);
    int r2 = r, k2 = k + 1;
    if (k2 >= cnt) {
      r2 = r + 1;
      k2 = 0;
    }
    const bool has_next = item_at(r2) < it_end;
    int nbh = bh, nkvh = kvh, nqblk = qblk;
    if (has_next) block_of(item_at(r2), k2, nbh, nkvh, nqblk);
    pre = fwd_block<D, CAUSAL, MASKED>(Q, K, V, O, LSE, Nq, Nk, sl2, bh, kvh, diag, qblk, n_qblk, kb0, kb1, vb0,
                                       vb1, stg, qf.f, pre, has_next, nbh, nkvh, nqblk, mk);
    r = r2;
    k = k2;
  }
}

// ------------------------------------------------------------------ fp32 path
// Same structure on v_mfma_f32_32x32x2_f32 (no down-conversion anywhere).  k-steps of
// S^T = K Q^T use the dim order k(t, h) = h*D/2 + t, so each lane reads contiguous float4s;
// the P V product takes one accumulator register per k-step, whose key is the accumulator
// row of that register, so no key permutation is needed.  LDS rows are padded by 16 bytes.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int Nq, int Nk, int n_qblk,
                                                      float sl2, int H, int group, int diag) {
  constexpr int BR = 128, BC = 32, RS = D + 4, HALF = D / 2, DBLK = D / 32;
  constexpr int TILE_FLOATS = BC * RS;
  constexpr int CH_PER_ROW = D / 4;
  constexpr int CHUNKS = BC * CH_PER_ROW / 256;
  __shared__ __attribute__((aligned(16))) float kt[TILE_FLOATS];
  __shared__ __attribute__((aligned(16))) float vt[TILE_FLOATS];

  int qblk = blockIdx.x % n_qblk;
  const int bh = blockIdx.x / n_qblk;
  if (CAUSAL) qblk = n_qblk - 1 - qblk;
  const int kvh = (bh / H) * (H / group) + (bh % H) / group;  // K/V head of query head bh
  const float* Qh = Q + (int64_t)bh * Nq * D;
  const float* Kh = K + (int64_t)kvh * Nk * D;
  const float* Vh = V + (int64_t)kvh * Nk * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int q_wave0 = qblk * BR + wave * 32;

  float qf[HALF];
  {
    const float* qp = Qh + (int64_t)min(q_wave0 + l32, Nq - 1) * D + hh * HALF;
#pragma unroll
    for (int i = 0; i < HALF; i += 4) {
      const f32x4_t x = *(const f32x4_t*)(qp + i);
      qf[i] = x[0]; qf[i + 1] = x[1]; qf[i + 2] = x[2]; qf[i + 3] = x[3];
    }
  }
  const int kv_end = CAUSAL ? min(Nk, qblk * BR + BR + diag) : Nk;
  const int n_tiles = (kv_end + BC - 1) / BC;

  f32x16_t oacc[DBLK];
#pragma unroll
  for (int mb = 0; mb < DBLK; ++mb) oacc[mb] = f32x16_t{};
  float m2 = -INFINITY, lsum = 0.f;

  for (int t = 0; t < n_tiles; ++t) {
    const int tile0 = t * BC;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int ci = tid + 256 * i, r = ci / CH_PER_ROW, c = ci % CH_PER_ROW;
      const int row = min(tile0 + r, Nk - 1);
      *(f32x4_t*)&kt[r * RS + 4 * c] = *(const f32x4_t*)(Kh + (int64_t)row * D + 4 * c);
      *(f32x4_t*)&vt[r * RS + 4 * c] = *(const f32x4_t*)(Vh + (int64_t)row * D + 4 * c);
    }
    __syncthreads();
    if (CAUSAL && tile0 > q_wave0 + 31 + diag) continue;
    f32x16_t s = f32x16_t{};
    const float* kr = &kt[l32 * RS + hh * HALF];
#pragma unroll
    for (int i = 0; i < HALF; i += 4) {
      const f32x4_t a = *(const f32x4_t*)(kr + i);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], qf[i], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], qf[i + 1], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], qf[i + 2], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], qf[i + 3], s, 0, 0, 0);
    }
    const bool need_mask = (tile0 + BC > Nk) || (CAUSAL && tile0 + BC - 1 > q_wave0 + diag);
    if (need_mask) {
      const int q = q_wave0 + l32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = tile0 + 8 * (j >> 2) + 4 * hh + (j & 3);
        if (key >= Nk || (CAUSAL && key > q + diag)) s[j] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
    mx = max_across_halves(mx);
    const float mnew = fmaxf(m2, mx * sl2);
    const float alpha = fast_exp2(m2 - mnew);
    m2 = mnew;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s[j] = fast_exp2(__builtin_fmaf(s[j], sl2, -mnew));
      rs += s[j];
    }
    lsum = alpha * lsum + rs;
#pragma unroll
    for (int mb = 0; mb < DBLK; ++mb) {
      oacc[mb] *= alpha;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int key = 8 * (u >> 2) + 4 * hh + (u & 3);
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[key * RS + 32 * mb + l32], s[u], oacc[mb], 0, 0, 0);
      }
    }
  }

  const float l = sum_across_halves(lsum);
  const float inv = 1.f / l;
  const int q = q_wave0 + l32;
  if (q < Nq) {
    float* op = O + (int64_t)bh * Nq * D + (int64_t)q * D + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < DBLK; ++mb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        f32x4_t w;
        w[0] = oacc[mb][4 * jg] * inv; w[1] = oacc[mb][4 * jg + 1] * inv;
        w[2] = oacc[mb][4 * jg + 2] * inv; w[3] = oacc[mb][4 * jg + 3] * inv;
        *(f32x4_t*)(op + 32 * mb + 8 * jg) = w;
      }
    if (hh == 0) LSE[(int64_t)bh * Nq + q] = (m2 + fast_log2(l)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool MASKED = false>
hipError_t launch_bf16_impl(const FwdArgs& a, hipStream_t stream) {
  using C = Bf16Cfg<D>;
  static_assert(C::BR == kFwdBlockRows, "the mask classification works on the forward's query blocks");
  const int n_qblk = (a.Nq + C::BR - 1) / C::BR;
  const int paired = (CAUSAL && (int64_t)a.B * a.H * ((n_qblk + 1) / 2) >= a.num_cus) ? 1 : 0;
  const int items_per_head = paired ? (n_qblk + 1) / 2 : n_qblk;
  const int64_t n_items = (int64_t)a.B * a.H * items_per_head;
  const int64_t grid = n_items < a.num_cus ? n_items : a.num_cus;
  const int xcd_split = (!MASKED && grid % 8 == 0 && n_items % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, MASKED>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     a.Nq, a.Nk, n_qblk, (int)n_items, items_per_head, xcd_split, a.scale * kLog2e, a.H,
                     a.H / a.H_kv, a.diag, paired, a.mask_counts, a.mask_lists, a.mask_words, a.mask_tiles,
                     a.mask_queue);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32_impl(const FwdArgs& a, hipStream_t stream) {
  const int n_qblk = (a.Nq + 127) / 128;
  const int64_t nblk = (int64_t)a.B * a.H * n_qblk;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nblk), dim3(256), 0, stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Nq, a.Nk,
                     n_qblk, a.scale * kLog2e, a.H, a.H / a.H_kv, a.diag);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_bf16_impl<128, true>(a, stream) : launch_bf16_impl<128, false>(a, stream);
  return a.causal ? launch_bf16_impl<64, true>(a, stream) : launch_bf16_impl<64, false>(a, stream);
}

hipError_t launch_fwd_bf16_masked(const FwdArgs& a, hipStream_t stream) {
  return a.d == 128 ? launch_bf16_impl<128, false, true>(a, stream) : launch_bf16_impl<64, false, true>(a, stream);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_f32_impl<128, true>(a, stream) : launch_f32_impl<128, false>(a, stream);
  return a.causal ? launch_f32_impl<64, true>(a, stream) : launch_f32_impl<64, false>(a, stream);
}

}  // namespace fa
