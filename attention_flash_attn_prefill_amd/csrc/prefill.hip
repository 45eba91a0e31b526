// Fused scaled-dot-product attention prefill for gfx950 (CDNA4, wave64).
//
// O = softmax(Q K^T * scale [+ causal mask]) V with an online (flash) softmax:
// the KV sequence is walked in tiles, a running row max and row sum are kept,
// and the output accumulator is rescaled when the max grows (flash-style
// attention as the pages' attention kernels compute it: "WAVE: A Symbolic
// Python DSL and Compiler for High Performance Machine Learning (MLSys 2026)",
// core method and attention experiments).
//
// Mapping onto the CDNA4 matrix cores
// -----------------------------------
// A workgroup owns 256 query rows of one (batch, head) (128 for D = 64); each
// of its eight (four) waves owns 32 of them, and all share each K/V tile.  The wave computes the *transposed* score tile
//     S^T (64 keys x 32 queries) = K (64 x D) . Q^T (D x 32)
// for each 64-key tile
// with v_mfma_f32_32x32x16_{f16,bf16}: K is the A operand (read from LDS), Q^T
// is the B operand (held in VGPRs for the whole KV loop).  In the 32x32 fp32
// accumulator a lane owns one query column (lane % 32) and 16 key rows, so
//   * the row max / row sum of a query is a reduction over the lane's own
//     registers plus one v_permlane32_swap with the partner lane (lane ^ 32),
//   * the rescale factor of a query is a per-lane scalar, and
//   * exp(S^T) rounded to fp16 is already laid out as the B operand of
//     O^T (D x 32) = V^T (D x 64) . P^T (64 x 32): P never round-trips
//     through LDS.
// The A operand V^T needs, per lane, eight keys of one d column of the
// row-major V tile: two ds_read_b64_tr_b16 per operand (CDNA4's transposing
// LDS read: within each 16-lane group, lane (r, c) names 4 halves of row r and
// lane j receives column j of the 4 x 16 block).
//
// Memory path: K and V tiles (64 keys x D) go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (no staging VGPRs, no ds_write, hardware range
// checking returns zeros past the sequence end), double-buffered so tile t+1
// streams in while tile t computes, with one barrier per tile (multi-buffering:
// "Wave February 2025 Release", Multi-Buffering list; 128-bit coalesced global
// reads: WAVE summary, lowering pipeline, global read coarsening; async
// global->LDS copies: "[FlyDSL] FP8 MQA logits improvements for gfx950",
// Changes / Kernel).  The 16-byte chunks of each LDS row are XOR-swizzled by a
// function of the row; the same XOR is applied to the DMA source address and
// to the read address, so it must be (and is) its own inverse.  For bf16
// inputs V is converted to fp16 on the way, so it is staged through VGPRs.
//
// Softmax numerics: scores stay fp32; the scale is folded in fp32 as
// c = scale*log2(e) into one FMA feeding v_exp_f32 (never into fp16/bf16 Q).
// The rescale is lazy: the reference max used in the exponent only moves
// when some row's max grows by more than 8 (in log2 units), so p <= 2^8 and
// most tiles skip the accumulator rescale.  The final O = acc / l is exact
// for any reference max.  P is rounded to fp16 (RNE) for both dtypes; for
// bf16 inputs V is converted to fp16 while it is staged (exact for
// 2^-14 <= |v| <= 65504), which keeps the bf16 output within 2e-3 relative
// Frobenius error of the exact result where bf16 P would not.
//
// Grid order: work items (b, h, query tile) are laid out so that consecutive
// workgroups on one XCD (workgroup i runs on XCD i % 8) take consecutive
// query tiles of the same head, sharing its K/V in that XCD's L2; causal grids
// run the heaviest query tiles first (workgroup reordering for L2 locality:
// WAVE summary, lowering pipeline).  Causal tiles wholly above the diagonal are
// never loaded, and only tiles that cross the diagonal or the sequence end are
// masked.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace mi355_attn {
namespace {

#include "cdna4_common.h"

// Extend batches of up to 64 * kExtMaxPerLane sequences are ordered longest
// unit first (wave 0 holds kExtMaxPerLane sequences per lane).
constexpr int kExtMaxPerLane = 8;

// NW waves per workgroup (BM = 32 * NW query rows), BN keys per KV tile.
// OF32: O is stored in fp32 instead of the input type.  EXT (with CAUSAL):
// extend attention -- a sequence's keys are its cached prefix, read through
// the page table, followed by its new tokens (PrefillArgs, extend fields).
// FP8: q, k, v are e4m3fn bytes; Q.K^T runs on the fp8 MFMA (32x32x64), V is
// widened to fp16 on staging, and BF16 then selects only the output type.
// SPLIT (with OF32, not EXT): the keys of each query tile are cut into
// a.n_splits ranges of a.split_tiles tiles, one work item each, which writes
// its partial O (normalised by its own row sums) and log-sum-exp into its
// split's planes of a.o and a.lse (flash decoding applied to prefill, for
// grids too small to fill the GPU); prefill_split_combine_kernel merges them.
template <int D, bool BF16, bool CAUSAL, bool OF32, int NW, int BN, bool EXT = false,
          bool FP8 = false, int HPW = 1, bool SPLIT = false>
__global__ __launch_bounds__(64 * NW, 2) void prefill_fwd_kernel(PrefillArgs a) {
  // The body uses amdgcn-only types (buffer resources, LDS address space); the
  // host pass only needs the kernel's signature for its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(!(EXT && FP8), "extend takes fp16/bf16");
  static_assert(!SPLIT || (OF32 && !FP8), "split partials are fp32; fp16/bf16 inputs");
  static_assert(NW % HPW == 0, "whole waves per query head");
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NW;
  constexpr int EB = FP8 ? 1 : 2;         // bytes per q/k/v element
  constexpr int CPR = D * EB / 16;        // 16-byte chunks per K/V row
  constexpr int LOADS = BN * CPR / NT;    // chunk loads per thread per K (or V) tile
  static_assert(LOADS * NT == BN * CPR, "tile must split evenly over the threads");
  static_assert(BN % 32 == 0 && 2 * 2 * BN * D * 2 <= 160 * 1024, "tile shape");
  static_assert(!EXT || (CAUSAL && BN % 16 == 0 && (64 / CPR) <= 16 && 16 % (64 / CPR) == 0),
                "extend: causal, and each load instruction's rows within one page");
  // Two LDS stages each of K and V, as separate objects so the compiler can
  // tell the stage being filled from the stage being read.
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[BN * D];
  // Extend: this workgroup's unit (sequence, query tile) and the sequence's
  // first row, new tokens and prefix length, when wave 0 has looked them up.
  __shared__ int ext_unit[5];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int li = lane & 31, hi = lane >> 5;

  // HPW query heads of one KV group per workgroup (1 or 4): the workgroup
  // covers RPW = BM / HPW rows of each, waves w*WPH .. w*WPH+WPH-1 taking
  // head w; every K/V tile staged in LDS then serves the HPW heads, and a
  // partial or causal query tile is RPW rows rather than BM.
  constexpr int RPW = BM / HPW, WPH = NW / HPW;
  // Work item L = ((b * H_kv + kv_head) * n_items + item) * (group / HPW) + gg:
  // the query heads that share a KV head are adjacent, so they run the same
  // query tile at the same time on one XCD and read the same K/V tiles
  // through its L2 (group = 1 is plain (b, h, item) order).
  //
  // Causal prefill over a large grid pairs the query tiles of a head: item p
  // runs query tile n - 1 - p (the heaviest left) and then tile p (the
  // lightest), so every workgroup walks about n + 1 tiles' worth of keys and
  // the grid has no tail of short workgroups (n = n_mtiles; the middle tile of
  // an odd n runs alone).  The launcher pairs only when the unpaired grid
  // fills the CUs at least twice (a.pair_tiles); a smaller grid would be left
  // with idle CUs.  Other work has one query tile per item, heaviest first.
  //
  // Extend batches are ragged.  With at most 512 sequences the work goes out
  // longest first over the whole batch: a unit is (sequence b, query tile
  // mt), worth ceil(P_b / RPW) + mt + 1 (its prefix plus causal keys, in
  // query-tile lengths), and units are taken in decreasing worth (ties by
  // sequence), each as H_kv * group / HPW adjacent workgroups (its KV heads
  // and head groups: with that a multiple of 8, a KV head always runs on the
  // same XCD).  The dispatcher hands an XCD's workgroups to its shader
  // engines in turn and in order, so heavy units last would leave engines
  // idle behind a long one.  Wave 0 finds this workgroup's unit from the
  // batch's sizes (lane l holding sequences l, 64 + l, ...): the unit's
  // worth c by bisection on the count of units worth at least c, then its
  // sequence among those with a unit worth exactly c.  Units past the last non-empty one have no
  // rows.  Larger batches go in (sequence, KV head) blocks interleaved over
  // the XCDs, heaviest query tile first within a block.
  const bool pairs = CAUSAL && !EXT && !SPLIT && a.pair_tiles;  // uniform
  const int hgroups = a.group / HPW;
  const int n_items = pairs ? (a.n_mtiles + 1) >> 1 : a.n_mtiles;
  int gg, item, hk, b;
  int split = 0;  // SPLIT: this work item's key range (workgroup-uniform)
  int e_r0 = 0, e_len = 0, e_pre = 0;  // sequence b's first row, new tokens, prefix
  bool e_known = false;                // whether those three are set (workgroup-uniform)
  if constexpr (EXT) {
    const int n_sp = SPLIT ? a.n_splits : 1;
    const int nb = a.total_tiles / (a.n_mtiles * hgroups * a.H_kv * n_sp);
    if (nb <= 64 * kExtMaxPerLane) {
      // SPLIT: a unit's key ranges follow its KV heads and head groups, so
      // the same KV head still lands on the same XCD.
      int L = blockIdx.x;
      gg = L % hgroups;
      L /= hgroups;
      hk = L % a.H_kv;
      L /= a.H_kv;
      if constexpr (SPLIT) {
        split = L % n_sp;
        L /= n_sp;
      }
      const int u = L;  // rank of the unit
      // Lane l holds sequences k * 64 + l, k < PER: their first row, new
      // tokens and prefix length (an invalid row range counts as no rows),
      // and their query tiles and prefix in query-tile lengths.  PER = 1 for
      // up to 64 sequences, kExtMaxPerLane beyond.
      auto find_unit = [&](auto per_c) __attribute__((always_inline)) {
        constexpr int PER = decltype(per_c)::value;
        int r0[PER], len[PER], pre[PER], nt[PER], npre[PER];
  #pragma unroll
        for (int k = 0; k < PER; ++k) {
          r0[k] = 0;
          len[k] = 0;
          pre[k] = 0;
          const int t = k * 64 + lane;
          if (t < nb) {
            r0[k] = a.qo_start[t];
            const int r1 = a.qo_start[t + 1];
            if (r0[k] >= 0 && r1 >= r0[k] && r1 <= a.total_tokens) {
              len[k] = min(r1 - r0[k], a.Sq);
              pre[k] = a.max_pages > 0
                           ? max(0, min(a.prefix_lens[t], a.max_pages * kDecodePageSize))
                           : 0;
            }
          }
          nt[k] = (len[k] + RPW - 1) / RPW;
          npre[k] = (pre[k] + RPW - 1) / RPW;
        }
        // Units of a sequence are worth npre + 1 .. npre + nt; at least c:
        auto count = [&](int c) __attribute__((always_inline)) {
          int n = 0;
  #pragma unroll
          for (int k = 0; k < PER; ++k) n += max(0, min(nt[k], npre[k] + nt[k] - c + 1));
          return wave_sum_i32(n);
        };
        int units = 0, top = 0;
  #pragma unroll
        for (int k = 0; k < PER; ++k) {
          units += nt[k];
          top = max(top, npre[k] + nt[k]);
        }
        int sel_b = -1, sel_mt = 0, sel_r0 = 0, sel_len = 0, sel_pre = 0;
        if (u < wave_sum_i32(units)) {
          int lo = 1, hi = wave_max_i32(top) + 1;  // count(lo) > u >= count(hi)
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (count(mid) > u) lo = mid;
            else hi = mid;
          }
          // Among the sequences with a unit worth lo (in sequence order),
          // this workgroup's is the j-th.
          int j = u - count(lo + 1);
  #pragma unroll
          for (int k = 0; k < PER; ++k) {
            if (sel_b >= 0) break;  // uniform
            const bool has = nt[k] > 0 && npre[k] < lo && lo <= npre[k] + nt[k];
            const uint64_t m = __builtin_amdgcn_read_exec() & __ballot(has);
            const int c = __builtin_popcountll(m);
            if (j >= c) {
              j -= c;
              continue;
            }
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const int pick = __builtin_ctzll(__ballot(has && below == j));
            sel_b = k * 64 + pick;
            sel_mt = lo - __builtin_amdgcn_readlane(npre[k], pick) - 1;
            sel_r0 = __builtin_amdgcn_readlane(r0[k], pick);
            sel_len = __builtin_amdgcn_readlane(len[k], pick);
            sel_pre = __builtin_amdgcn_readlane(pre[k], pick);
          }
        }
        if (lane == 0) {
          ext_unit[0] = sel_b;
          ext_unit[1] = sel_mt;
          ext_unit[2] = sel_r0;
          ext_unit[3] = sel_len;
          ext_unit[4] = sel_pre;
        }
      };
      if (wave == 0) {
        if (nb <= 64) find_unit(std::integral_constant<int, 1>{});
        else find_unit(std::integral_constant<int, kExtMaxPerLane>{});
      }
      __syncthreads();
      b = __builtin_amdgcn_readfirstlane(ext_unit[0]);
      const int mt = __builtin_amdgcn_readfirstlane(ext_unit[1]);
      if (b < 0 || b >= nb || mt < 0 || mt >= a.n_mtiles) return;  // no rows (workgroup-uniform)
      item = a.n_mtiles - 1 - mt;  // the part loop takes query tile n_mtiles - 1 - item
      e_r0 = __builtin_amdgcn_readfirstlane(ext_unit[2]);
      e_len = __builtin_amdgcn_readfirstlane(ext_unit[3]);
      e_pre = __builtin_amdgcn_readfirstlane(ext_unit[4]);
      e_known = true;
    } else {
      int w = (int)blockIdx.x;
      if constexpr (SPLIT) {
        split = w % n_sp;
        w /= n_sp;
      }
      int L = xcd_interleave(w, a.total_tiles / (a.n_mtiles * hgroups * n_sp),
                             a.n_mtiles * hgroups);
      gg = L % hgroups;
      L /= hgroups;
      item = L % n_items;
      L /= n_items;
      hk = L % a.H_kv;
      b = L / a.H_kv;
    }
  } else {
    int L = xcd_remap(blockIdx.x, a.total_tiles);
    if constexpr (SPLIT) {  // the splits of a query tile are adjacent (one XCD)
      split = L % a.n_splits;
      L /= a.n_splits;
    }
    gg = L % hgroups;
    L /= hgroups;
    item = L % n_items;
    L /= n_items;
    hk = L % a.H_kv;
    b = L / a.H_kv;
  }
  const int h = hk * a.group + gg * HPW + wave / WPH;  // wave-uniform
  const int n_parts = (pairs && a.n_mtiles - 1 - item != item) ? 2 : 1;

  for (int part = 0; part < n_parts; ++part) {
    // Query tile of this part: extend in order; causal heaviest first.
    const int mt = !CAUSAL ? item : (pairs && part == 1 ? item : a.n_mtiles - 1 - item);
    // The second part refills the LDS stages: every wave must be done with
    // the first part's last tile.
    if (part > 0) __syncthreads();

    // Sequence sizes.  Extend: Sq = the sequence's new tokens, Skv = prefix +
    // new, bottom-right causal (offset = prefix length); the first n_pre tiles
    // hold prefix keys [0, P) from the cache, the rest new keys from k, v.
    int Sq = a.Sq, Skv = a.Skv, coff = a.causal_off, P = 0, n_pre = 0;
    int row0 = 0;  // extend: the sequence's first row of q, k, v, o
    int64_t q_base = b * a.q_sb + h * a.q_sh;   // o shares q's element strides
    int64_t kv_base = b * a.k_sb + hk * a.k_sh;
    if constexpr (EXT) {
      int r0 = e_r0;
      if (e_known) {
        Sq = e_len;
        P = e_pre;
      } else {
        r0 = a.qo_start[b];
        const int r1 = a.qo_start[b + 1];
        if (r0 < 0 || r1 < r0 || r1 > a.total_tokens) return;  // invalid range: not computed
        Sq = min(r1 - r0, a.Sq);                                // a.Sq = max_extend_len
        P = a.max_pages > 0 ? max(0, min(a.prefix_lens[b], a.max_pages * kDecodePageSize)) : 0;
      }
      Skv = P + Sq;
      coff = P;
      n_pre = (P + BN - 1) / BN;
      row0 = r0;
      q_base = (int64_t)r0 * a.q_ss + h * a.q_sh;
      kv_base = (int64_t)r0 * a.k_ss + hk * a.k_sh;
    }
    const char* __restrict__ qp = reinterpret_cast<const char*>(a.q) + q_base * EB;
    const int64_t o_base = q_base;
    const char* __restrict__ kp = reinterpret_cast<const char*>(a.k) + kv_base * EB;
    const char* __restrict__ vp = reinterpret_cast<const char*>(a.v) + kv_base * EB;

    const int m0 = mt * RPW;
    if (EXT && m0 >= Sq) return;  // past this sequence's new tokens (workgroup-uniform)
    const int q0 = m0 + (wave % WPH) * 32;
    const int qi = q0 + li;
    const bool q_ok = qi < Sq;

    // Q^T fragments (B operand): lane holds Q[qi][16s + 8hi .. +7] (16-bit), or
    // Q[qi][64s + 32hi .. +31] (fp8).
    constexpr int QF = FP8 ? 1 : D / 16;
    constexpr int QF8 = FP8 ? D / 64 : 1;
    u32x4 qf[QF];
    i32x8 qf8[QF8];
    const char* qrow = qp + (int64_t)qi * a.q_ss * EB;
    if constexpr (FP8) {
  #pragma unroll
      for (int s = 0; s < QF8; ++s) {
        const u32x4 lo = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 64 * s + 32 * hi)
                              : (u32x4){0u, 0u, 0u, 0u};
        const u32x4 up = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 64 * s + 32 * hi + 16)
                              : (u32x4){0u, 0u, 0u, 0u};
        qf8[s] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
      }
    } else {
  #pragma unroll
      for (int s = 0; s < QF; ++s)
        qf[s] = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 2 * (16 * s + 8 * hi))
                     : (u32x4){0u, 0u, 0u, 0u};
    }

    // Keys this workgroup needs: [0, kv_end).
    int kv_end = Skv;
    if (CAUSAL) kv_end = min(kv_end, max(0, min(m0 + RPW, Sq) + coff));
    // SPLIT: this work item takes key tiles [kt0, kt0 + n_tiles) of them.
    int kt0 = 0;
    int n_tiles = EXT ? n_pre + (kv_end - P + BN - 1) / BN : (kv_end + BN - 1) / BN;
    if constexpr (SPLIT) {
      kt0 = split * a.split_tiles;
      n_tiles = max(0, min(n_tiles, kt0 + a.split_tiles) - kt0);
    }
    // Keys this wave needs: [0, wave_kv_end).
    const bool wave_active = q0 < Sq;
    const int wave_kv_end = CAUSAL ? min(Skv, min(q0 + 32, Sq) + coff) : Skv;
    // Tile t of this work item is tile gtile(t) of the item's keys; its first
    // key (in the whole key sequence), and whether it is a prefix tile
    // (extend only).
    auto gtile = [&](int t) { return SPLIT ? kt0 + t : t; };
    auto is_pre = [&](int t) { return EXT && gtile(t) < n_pre; };
    auto tile_key0 = [&](int t) {
      const int g = gtile(t);
      return EXT ? (g < n_pre ? g * BN : P + (g - n_pre) * BN) : g * BN;
    };

    // ---- K/V staging addresses (loop invariant).  Load i of this thread fills
    // LDS chunk P = (wave * LOADS + i) * 64 + lane of the tile: row P / CPR,
    // position P % CPR, holding logical chunk position ^ swz(row).
    int g_off[LOADS];  // byte offset of the chunk within the tile's rows
  #pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int chunk = (wave * LOADS + i) * 64 + lane;
      const int row = chunk / CPR, pos = chunk % CPR;
      if constexpr (FP8)
        g_off[i] = row * a.k_ss + (pos ^ swz_fp8<D>(row)) * 16;
      else
        g_off[i] = (row * a.k_ss + ((pos ^ swz<D>(row)) * 8)) * 2;
    }
    const uint32_t row_bytes = (uint32_t)a.k_ss * EB;
    const int n_rows = EXT ? Sq : Skv;  // rows of k, v (the new tokens, for extend)

    auto tile_rsrc = [&](const char* base, int kv0) {
      const uint32_t rows = (uint32_t)max(0, n_rows - kv0);
      return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * a.k_ss * EB), (short)0,
                                               (int)(rows * row_bytes), kBufferConfig);
    };

    // Extend prefix tiles: the loads of a wave cover its WAVE_ROWS rows of the
    // tile, which lie in one page (page wpage of the tile; pages hold 16
    // tokens), so one buffer per tile and cache serves them all.  It spans the
    // page's slots below P, so rows past the prefix read as zero.
    constexpr int ROWS_PER_LOAD = 64 / CPR;
    constexpr int WAVE_ROWS = LOADS * ROWS_PER_LOAD;
    static_assert(!EXT || kDecodePageSize % WAVE_ROWS == 0, "a wave's rows of a tile in one page");
    const int wpage = (wave * WAVE_ROWS) / kDecodePageSize;  // wave-uniform
    const int64_t page_elems = (int64_t)kDecodePageSize * a.H_kv * D;
    const uint32_t slot_bytes = (uint32_t)a.H_kv * D * 2u;
    const int32_t* ptab = EXT ? a.page_table + (int64_t)b * a.max_pages : nullptr;
    int pg_off[LOADS];  // byte offset of the chunk within its page
    if constexpr (EXT) {
  #pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int chunk = (wave * LOADS + i) * 64 + lane;
        const int row = chunk / CPR, pos = chunk % CPR;
        pg_off[i] = ((row % kDecodePageSize) * a.H_kv * D + hk * D + ((pos ^ swz<D>(row)) * 8)) * 2;
      }
    }
    bool bad_page = false;  // workgroup-uniform: a prefix page id outside the pool
    // Page ids of the next prefix tile to load (0 where the tile holds no live
    // token: such a page is never read), fetched a tile ahead by a vector load
    // -- lane j & 3 reads page j of the tile -- so the read is waited for with
    // the tile loads (vmcnt) at the next barrier; a scalar load would share its
    // counter with the LDS operand reads and stall the compute in between.
    constexpr int PPT = BN / kDecodePageSize;  // pages per tile
    static_assert(PPT == 4, "page ids of a tile are held by lanes j & 3");
    int pgv_next = 0;
    auto fetch_pages = [&](int t) {
      const int tok = gtile(t) * BN + (lane & 3) * kDecodePageSize;
      pgv_next = (EXT && gtile(t) < n_pre && tok < P) ? ptab[tok / kDecodePageSize] : 0;
    };
    // Every wave checks every page of the tile (as unsigned, so negative ids
    // are rejected too), so all waves agree.
    auto pages_ok = [&]() {
      return __builtin_amdgcn_ballot_w64((uint32_t)pgv_next >= (uint32_t)a.num_pages) == 0;
    };
    // Buffers of this wave's page of the tile being loaded, in the K and the V
    // cache.  The range is wave-uniform; keeping it in an SGPR keeps the
    // compiler from wrapping every load in a waterfall loop over the lanes (it
    // would otherwise clamp it with a vector instruction).
    __amdgpu_buffer_rsrc_t pk_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.k_cache, (short)0, 0, kBufferConfig);
    __amdgpu_buffer_rsrc_t pv_rsrc = pk_rsrc;
    auto set_page_rsrc = [&](int t) {
      const int live = min(kDecodePageSize, P - (gtile(t) * BN + wpage * kDecodePageSize));
      const int64_t off = live > 0 ? (int64_t)__builtin_amdgcn_readlane(pgv_next, wpage) * page_elems
                                   : 0;
      const int nbytes = __builtin_amdgcn_readfirstlane(max(live, 0) * (int)slot_bytes);
      pk_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_cache + off), (short)0, nbytes,
                                                  kBufferConfig);
      pv_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v_cache + off), (short)0, nbytes,
                                                  kBufferConfig);
    };

    // DMA loads of one K tile, and of one V tile (for bf16, V goes to registers
    // first for the fp16 conversion; store_v writes it to LDS).
    u32x4 vreg[LOADS];
    auto issue_k = [&](int t, LDS_AS uint16_t* k_dst) {
      if (is_pre(t)) {
  #pragma unroll
        for (int i = 0; i < LOADS; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(pk_rsrc,
                                                   (LDS_AS void*)(k_dst + (wave * LOADS + i) * 512),
                                                   16, pg_off[i], 0, 0, 0);
        return;
      }
      const auto rk = tile_rsrc(kp, tile_key0(t) - P);
  #pragma unroll
      for (int i = 0; i < LOADS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS_AS void*)(k_dst + (wave * LOADS + i) * 512),
                                                 16, g_off[i], 0, 0, 0);
    };
    auto issue_v = [&](int t, LDS_AS uint16_t* v_dst) {
      const bool pre = is_pre(t);
      const auto rv = tile_rsrc(vp, pre ? 0 : tile_key0(t) - P);
  #pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const auto r = pre ? pv_rsrc : rv;
        const int off = pre ? pg_off[i] : g_off[i];
        if constexpr (BF16 || FP8)
          vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(v_dst + (wave * LOADS + i) * 512),
                                                   16, off, 0, 0, 0);
      }
    };
    // fp8: widen the staged V chunk (16 e4m3fn values of row r, logical chunk
    // c) to fp16 and write its two fp16 chunks 2c, 2c+1 of row r to LDS.
    // bf16: convert the staged V chunks to fp16 and write them to LDS.
    auto store_v = [&](LDS_AS uint16_t* v_dst) {
      if constexpr (FP8) {
  #pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int chunk = (wave * LOADS + i) * 64 + lane;
          const int row = chunk / CPR, c = (chunk % CPR) ^ swz_fp8<D>(row);
          u32x4 w[2];
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x2 h = fp8x4_to_f16x4(vreg[i][j]);
            w[j >> 1][2 * (j & 1)] = h[0];
            w[j >> 1][2 * (j & 1) + 1] = h[1];
          }
  #pragma unroll
          for (int u = 0; u < 2; ++u)
            *reinterpret_cast<LDS_AS u32x4*>(v_dst + row * D + (((2 * c + u) ^ swz<D>(row)) * 8)) =
                w[u];
        }
      } else if constexpr (BF16) {
  #pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int base = (wave * LOADS + i) * 64 * 8 + lane * 8;
          u32x4 w;
  #pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = bf16x2_to_f16x2(vreg[i][j]);
          *reinterpret_cast<LDS_AS u32x4*>(v_dst + base) = w;
        }
      }
    };

    // ---- LDS read offsets (halves, loop invariant).
    // K (A operand of S^T): lane reads row 32jb + li, logical chunk 2s + hi.
    // fp8: lane reads row 32jb + li, logical chunks 4s + 2hi and +1 (halves
    // offsets into rows of D bytes).
    int k_rd[FP8 ? 2 * (D / 64) : D / 16];
    if constexpr (FP8) {
  #pragma unroll
      for (int s = 0; s < D / 64; ++s)
  #pragma unroll
        for (int u = 0; u < 2; ++u)
          k_rd[2 * s + u] = (li * D + (((4 * s + 2 * hi + u) ^ swz_fp8<D>(li)) * 16)) / 2;
    } else {
  #pragma unroll
      for (int s = 0; s < D / 16; ++s) k_rd[s] = li * D + (((2 * s + hi) ^ swz<D>(li)) * 8);
    }
    // V (transposing reads): lane (group g = lane/16, r, c) names 4 halves of
    // key 16s + 8half + 4hi + r at d = 32db + 16(g & 1) + 4c.
    const int g16 = lane >> 4, tr_r = (lane >> 2) & 3, tr_c = lane & 3;
    int v_rd[2][D / 32];
  #pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int key = 8 * half + 4 * hi + tr_r;  // key within its 16-key step (key & 15)
  #pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int chunk = 4 * db + 2 * (g16 & 1) + (tr_c >> 1);
        v_rd[half][db] = key * D + ((chunk ^ swz<D>(key)) * 8) + (tr_c & 1) * 4;
      }
    }

    f32x16 acc[D / 32];
  #pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
    float m_run = kNegInf;  // reference max (log2 units) used in the exponent
    float l_run = 0.f;      // this lane's share of the row sum

    // ---- per-tile pieces.

    // S^T = K Q^T for one tile: one 32-key accumulator chain per 32 keys,
    // interleaved.
    auto qk = [&](const LDS_AS uint16_t* ks, f32x16 (&sc)[BN / 32]) {
      if constexpr (FP8) {
        // Rows of D bytes: block jb starts at byte 32 jb D.
        i32x8 kf8[D / 64][BN / 32];
  #pragma unroll
        for (int s = 0; s < D / 64; ++s)
  #pragma unroll
          for (int jb = 0; jb < BN / 32; ++jb) {
            const u32x4 lo = *reinterpret_cast<const LDS_AS u32x4*>(ks + 16 * jb * D + k_rd[2 * s]);
            const u32x4 up = *reinterpret_cast<const LDS_AS u32x4*>(ks + 16 * jb * D + k_rd[2 * s + 1]);
            kf8[s][jb] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
          }
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int jb = 0; jb < BN / 32; ++jb) sc[jb] = (f32x16){};
  #pragma unroll
        for (int s = 0; s < D / 64; ++s)
  #pragma unroll
          for (int jb = 0; jb < BN / 32; ++jb) sc[jb] = mfma_qk_fp8(kf8[s][jb], qf8[s], sc[jb]);
        return;
      }
      // All K fragments are read before the first MFMA (the fence keeps the
      // scheduler from recycling two registers and exposing an LDS round trip
      // per MFMA pair).
      u32x4 kf[D / 16][BN / 32];
  #pragma unroll
      for (int s = 0; s < D / 16; ++s)
  #pragma unroll
        for (int jb = 0; jb < BN / 32; ++jb)
          kf[s][jb] = *reinterpret_cast<const LDS_AS u32x4*>(ks + 32 * jb * D + k_rd[s]);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int jb = 0; jb < BN / 32; ++jb) sc[jb] = (f32x16){};
  #pragma unroll
      for (int s = 0; s < D / 16; ++s)
  #pragma unroll
        for (int jb = 0; jb < BN / 32; ++jb) sc[jb] = mfma_qk<BF16>(kf[s][jb], qf[s], sc[jb]);
    };

    // Mask keys past the sequence end and (causal) above the diagonal; in an
    // extend prefix tile, the rows past the prefix.
    auto mask_tile = [&](int t, f32x16 (&sc)[BN / 32]) {
      const int kv0 = tile_key0(t);
      const bool pre = is_pre(t);
      const bool need_mask = pre ? kv0 + BN > P
                                 : (kv0 + BN > Skv) || (CAUSAL && kv0 + BN - 1 > q0 + coff);
      if (need_mask) {
        const int lim = pre ? P - 1 : (CAUSAL ? min(Skv - 1, qi + coff) : Skv - 1);
  #pragma unroll
        for (int jb = 0; jb < BN / 32; ++jb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * jb + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key > lim) sc[jb][r] = kNegInf;
          }
      }
    };

    // Row max over the tile's keys and the lazy rescale; returns the
    // reference max used in this tile's exponent.
    auto max_rescale = [&](const f32x16 (&sc)[BN / 32]) {
      float mx = kNegInf;
  #pragma unroll
      for (int jb = 0; jb < BN / 32; ++jb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[jb][r]);
      mx = pair_max(mx) * a.c;
      // Move the reference max only when some row's max grew by more than 8.
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
  #pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
        m_run = m_new;
      }
      return (m_run == kNegInf) ? 0.f : m_run;
    };

    // P^T = exp2(S^T * c - base) rounded to fp16 (the B operand of P.V), and
    // the row sum of exactly those rounded values.
    auto exp_tile = [&](const f32x16 (&sc)[BN / 32], float base, u32x4 (&pf)[BN / 16]) {
  #pragma unroll
      for (int s = 0; s < BN / 16; ++s) {
        float e[8];
  #pragma unroll
        for (int j = 0; j < 8; ++j)
          e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[s >> 1][8 * (s & 1) + j], a.c, -base));
        // Keep the pairs as f16x2 values: clang lowers a bit-cast of an
        // ext-vector *element* (pf[s][j]) as a read of element 0.
        f16x2 hp[4];
  #pragma unroll
        for (int j = 0; j < 4; ++j)
          hp[j] = __builtin_convertvector((f32x2){e[2 * j], e[2 * j + 1]}, f16x2);
        pf[s] = (u32x4){__builtin_bit_cast(uint32_t, hp[0]), __builtin_bit_cast(uint32_t, hp[1]),
                        __builtin_bit_cast(uint32_t, hp[2]), __builtin_bit_cast(uint32_t, hp[3])};
  #pragma unroll
        for (int j = 0; j < 4; ++j)
          l_run = __builtin_amdgcn_fdot2(hp[j], (f16x2){(_Float16)1.0f, (_Float16)1.0f}, l_run,
                                         false);
      }
    };

    // O^T += V^T P^T ; V^T operand = two transposing reads (keys +0..3, +8..11
    // of the lane half's 16-key step).
    auto pv = [&](const u32x4 (&pf)[BN / 16], const LDS_AS uint16_t* vs) {
      // All V^T fragments are read before the first MFMA (see qk).
      u32x4 vf[BN / 16][D / 32];
  #pragma unroll
      for (int s = 0; s < BN / 16; ++s)
  #pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
              (LDS_AS fp16x4_t*)(vs + 16 * s * D + v_rd[0][db]));
          const fp16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
              (LDS_AS fp16x4_t*)(vs + 16 * s * D + v_rd[1][db]));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
          const u32x2 h2 = __builtin_bit_cast(u32x2, hi4);
          vf[s][db] = (u32x4){l2[0], l2[1], h2[0], h2[1]};
        }
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int s = 0; s < BN / 16; ++s)
  #pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma_pv(vf[s][db], pf[s], acc[db]);
    };

    // ---- main loop: two LDS stages; tile t+1 streams in while tile t
    // computes; one barrier per tile.
    LDS_AS uint16_t* const Ks[2] = {(LDS_AS uint16_t*)k_lds0, (LDS_AS uint16_t*)k_lds1};
    LDS_AS uint16_t* const Vs[2] = {(LDS_AS uint16_t*)v_lds0, (LDS_AS uint16_t*)v_lds1};

    // A tile is loaded only when its pages check out (dense tiles always do);
    // its page buffers are set up and the following tile's ids are fetched.
    auto load_ok = [&](int t) {
      if constexpr (EXT) {
        if (is_pre(t)) {
          if (!pages_ok()) bad_page = true;
          else set_page_rsrc(t);
        }
        fetch_pages(t + 1);
      }
      return !bad_page;
    };
    if constexpr (EXT) fetch_pages(0);
    if (n_tiles > 0 && load_ok(0)) {
      issue_v(0, Vs[0]);
      issue_k(0, Ks[0]);
      store_v(Vs[0]);
    }
    auto iteration = [&](int t, auto par) {
      constexpr int S = decltype(par)::value;  // t % 2
      // Tile t has landed for this wave; after the barrier for every wave, and
      // every wave is done with tile t-1, whose stages are refilled next.
      wait_vmcnt<0>();
      __syncthreads();
      const bool more = t + 1 < n_tiles && load_ok(t + 1);
      if (more) {
        issue_v(t + 1, Vs[S ^ 1]);
        issue_k(t + 1, Ks[S ^ 1]);
      }
      if (wave_active && (is_pre(t) || tile_key0(t) < wave_kv_end)) {
        f32x16 sc[BN / 32];
        qk(Ks[S], sc);
        mask_tile(t, sc);
        const float base = max_rescale(sc);
        u32x4 pf[BN / 16];
        exp_tile(sc, base, pf);
        pv(pf, Vs[S]);
      }
      if (more) store_v(Vs[S ^ 1]);
    };
    for (int t = 0; t < n_tiles; t += 2) {
      iteration(t, std::integral_constant<int, 0>{});
      if (t + 1 < n_tiles) iteration(t + 1, std::integral_constant<int, 1>{});
    }

    // Epilogue: O = acc / l.  Lane owns query qi and, in block db, the four
    // consecutive d = 32db + 8g + 4hi .. +3 for g = 0..3.
    const float l_tot = pair_sum(l_run);
    // SPLIT: the work item's planes of the partial outputs.
    float* const lse_out = SPLIT ? a.lse + split * a.split_lse_stride : a.lse;
    void* const o_out = SPLIT ? static_cast<void*>(static_cast<float*>(a.o) + split * a.split_o_stride)
                              : a.o;
    if (lse_out != nullptr && q_ok && hi == 0) {
      // log2-sum-exp of s c is m_run + log2(l); the natural one of s scale is
      // that times ln 2.  A split that met a rejected prefix page passes NaN
      // on, so the merged row is NaN too.  Split extend rows are token-major:
      // the log-sum-exps are [H, total_tokens].
      const float lse2 = (SPLIT && bad_page) ? __builtin_nanf("")
                         : l_tot > 0.f       ? m_run + __log2f(l_tot)
                                             : kNegInf;
      const int64_t li_row = (EXT && SPLIT) ? (int64_t)h * a.total_tokens + row0 + qi
                                            : ((int64_t)b * a.H + h) * Sq + qi;
      lse_out[li_row] = lse2 * 0.6931471805599453f;
    }
    // A rejected prefix page makes the rows NaN (the key set is unknown).
    const float inv =
        bad_page ? __builtin_nanf("") : (l_tot > 0.f ? a.o_scale / l_tot : 0.f);
    if (q_ok) {
      const int64_t row = o_base + (int64_t)qi * a.q_ss;
  #pragma unroll
      for (int db = 0; db < D / 32; ++db)
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float* v4 = reinterpret_cast<const float*>(&acc[db]) + 4 * g;
          const int d0 = 32 * db + 8 * g + 4 * hi;
          if constexpr (OF32) {
            const f32x4 out = {v4[0] * inv, v4[1] * inv, v4[2] * inv, v4[3] * inv};
            *reinterpret_cast<f32x4*>(static_cast<float*>(o_out) + row + d0) = out;
          } else {
            u32x2 out;
            if constexpr (BF16) {
              out[0] = pack_bf16(v4[0] * inv, v4[1] * inv);
              out[1] = pack_bf16(v4[2] * inv, v4[3] * inv);
            } else {
              out[0] = pack_f16(v4[0] * inv, v4[1] * inv);
              out[1] = pack_f16(v4[2] * inv, v4[3] * inv);
            }
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o_out) + row + d0) = out;
          }
        }
    }
  }  // part
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool BF16, bool CAUSAL, bool OF32, int NW, int BN, bool EXT = false,
          bool FP8 = false, int HPW = 1>
hipError_t launch_t(PrefillArgs a, int B, hipStream_t s) {
  constexpr int RPW = 32 * NW / HPW;  // query rows per head in a workgroup
  const int64_t n_mtiles = (a.Sq + RPW - 1) / RPW;
  // Causal prefill: one workgroup per pair of query tiles (see the kernel)
  // when the unpaired grid covers the GPU's 256 CUs at least twice.
  const int64_t unpaired = (int64_t)B * (a.H / HPW) * n_mtiles;
  a.pair_tiles = (CAUSAL && !EXT && unpaired >= 2 * kNumCUs) ? 1 : 0;
  const int64_t n_items = a.pair_tiles ? (n_mtiles + 1) / 2 : n_mtiles;
  const int64_t total = (int64_t)B * (a.H / HPW) * n_items;
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  a.n_mtiles = (int)n_mtiles;
  a.total_tiles = (int)total;
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, CAUSAL, OF32, NW, BN, EXT, FP8, HPW>),
                     dim3(a.total_tiles), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// Four query heads per workgroup when the KV group allows it (group % 4 == 0),
// for causal and extend work, where the shorter query tiles pay.
template <int D, bool BF16, bool CAUSAL, bool OF32, int NW, int BN, bool EXT = false>
hipError_t launch_g(const PrefillArgs& a, int B, hipStream_t s) {
  if ((CAUSAL || EXT) && a.group % 4 == 0)
    return launch_t<D, BF16, CAUSAL, OF32, NW, BN, EXT, false, 4>(a, B, s);
  return launch_t<D, BF16, CAUSAL, OF32, NW, BN, EXT, false, 1>(a, B, s);
}

// D = 128: eight waves (256 query rows) share each 64-key K/V tile, one
// workgroup per CU (two waves per SIMD); D = 64: four waves (128 rows).
template <int D, bool BF16, bool OF32>
hipError_t launch_c(bool causal, const PrefillArgs& a, int B, hipStream_t s) {
  constexpr int NW = D == 128 ? 8 : 4;
  constexpr int BN = 64;
  return causal ? launch_g<D, BF16, true, OF32, NW, BN>(a, B, s)
                : launch_t<D, BF16, false, OF32, NW, BN>(a, B, s);
}

template <int D, bool OF32>
hipError_t launch_d(bool bf16, bool causal, const PrefillArgs& a, int B, hipStream_t s) {
  return bf16 ? launch_c<D, true, OF32>(causal, a, B, s)
              : launch_c<D, false, OF32>(causal, a, B, s);
}

template <int D>
hipError_t launch_o(bool bf16, bool causal, bool out_f32, const PrefillArgs& a, int B,
                    hipStream_t s) {
  return out_f32 ? launch_d<D, true>(bf16, causal, a, B, s)
                 : launch_d<D, false>(bf16, causal, a, B, s);
}

}  // namespace

hipError_t launch_prefill(int D, bool bf16, bool causal, bool out_f32, const PrefillArgs& a,
                          int B, hipStream_t s) {
  if (D == 128) return launch_o<128>(bf16, causal, out_f32, a, B, s);
  if (D == 64) return launch_o<64>(bf16, causal, out_f32, a, B, s);
  return hipErrorInvalidValue;
}

namespace {

// Merge of one query row's split-KV partials: the mean of the splits'
// normalised partial rows weighted by exp(lse_s - max lse).  A row no split
// saw (every lse_s = -inf) gets O = 0; a row with a NaN log-sum-exp (a split
// that met a rejected prefix page, or NaN inputs) gets NaN.  Eight lanes per
// row: lane k of the row owns the D/8 consecutive outputs at element `off`
// of o (and of each partial plane); lrow indexes the log-sum-exp planes.
template <int D, bool BF16, bool OF32>
__device__ __forceinline__ void merge_split_row(const PrefillArgs& a, const float* part_o,
                                                const float* part_lse, int64_t lrow,
                                                int64_t off) {
  constexpr int E = D / 8;  // outputs per lane
  constexpr float kLog2e = 1.4426950408889634f;
  float m = kNegInf;
  bool nan = false;
  for (int sp = 0; sp < a.n_splits; ++sp) {
    const float x = part_lse[sp * a.split_lse_stride + lrow];
    nan |= x != x;
    m = fmaxf(m, x);
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m != kNegInf && !nan) {
    for (int sp = 0; sp < a.n_splits; ++sp) {
      const float w =
          __builtin_amdgcn_exp2f((part_lse[sp * a.split_lse_stride + lrow] - m) * kLog2e);
      const f32x4* src = reinterpret_cast<const f32x4*>(part_o + sp * a.split_o_stride + off);
      wsum += w;
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        const f32x4 x = src[c];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * c + j] = __builtin_fmaf(w, x[j], acc[4 * c + j]);
      }
    }
  }
  const float inv = nan ? __builtin_nanf("") : (wsum > 0.f ? 1.f / wsum : 0.f);
  if constexpr (OF32) {
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + off);
#pragma unroll
    for (int c = 0; c < E / 4; ++c)
      dst[c] = (f32x4){acc[4 * c] * inv, acc[4 * c + 1] * inv, acc[4 * c + 2] * inv,
                       acc[4 * c + 3] * inv};
  } else {
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + off);
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      u32x4 w4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = acc[8 * c + 2 * j] * inv, x1 = acc[8 * c + 2 * j + 1] * inv;
        w4[j] = BF16 ? pack_bf16(x0, x1) : pack_f16(x0, x1);
      }
      dst[c] = w4;
    }
  }
}

// Combine of split-KV prefill: query row (b, h, i) is row (b * H + h) * Sq + i
// of the log-sum-exp planes; eight rows per 64-lane workgroup.
template <int D, bool BF16, bool OF32>
__global__ __launch_bounds__(64) void prefill_split_combine_kernel(PrefillArgs a, int B,
                                                                   const float* part_o,
                                                                   const float* part_lse) {
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * 8 + (lane >> 3);
  if (row >= (int64_t)B * a.H * a.Sq) return;  // whole 8-lane groups leave together
  const int qi = (int)(row % a.Sq);
  const int64_t bh = row / a.Sq;
  const int h = (int)(bh % a.H);
  const int64_t b = bh / a.H;
  const int64_t off = b * a.q_sb + h * a.q_sh + (int64_t)qi * a.q_ss + (lane & 7) * (D / 8);
  merge_split_row<D, BF16, OF32>(a, part_o, part_lse, row, off);
}

// Combine of split-KV extend: workgroup (x, y) merges rows 8 * (x / H) ..
// +7 of query head x % H of sequence y, each the token qo_start[y] + i, row
// h * total_tokens + token of the log-sum-exp planes.  It writes exactly the
// rows the extend kernel computes: those of a sequence whose qo_start range
// lies in [0, total_tokens], below max_extend_len (a.Sq).
template <int D, bool BF16, bool OF32>
__global__ __launch_bounds__(64) void extend_split_combine_kernel(PrefillArgs a,
                                                                  const float* part_o,
                                                                  const float* part_lse) {
  const int lane = threadIdx.x;
  const int b = blockIdx.y;
  const int h = (int)(blockIdx.x % (unsigned)a.H);
  const int i = (int)(blockIdx.x / (unsigned)a.H) * 8 + (lane >> 3);
  const int r0 = a.qo_start[b], r1 = a.qo_start[b + 1];
  if (r0 < 0 || r1 < r0 || r1 > a.total_tokens) return;  // not computed
  if (i >= min(r1 - r0, a.Sq)) return;                    // whole 8-lane groups
  const int64_t tok = (int64_t)r0 + i;
  const int64_t off = tok * a.q_ss + h * a.q_sh + (lane & 7) * (D / 8);
  merge_split_row<D, BF16, OF32>(a, part_o, part_lse, (int64_t)h * a.total_tokens + tok, off);
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_split_t(const PrefillArgs& a, int B, float* part_o, float* part_lse,
                          bool out_f32, hipStream_t s) {
  constexpr int NW = D == 128 ? 8 : 4;
  constexpr int BN = 64;
  constexpr int RPW = 32 * NW;
  const int64_t n_mtiles = (a.Sq + RPW - 1) / RPW;
  const int64_t total = (int64_t)B * a.H * n_mtiles * a.n_splits;
  const int64_t rows = (int64_t)B * a.H * a.Sq;
  if (total >= ((int64_t)1 << 31) || (rows + 7) / 8 >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  PrefillArgs p = a;
  p.o = part_o;
  p.lse = part_lse;
  p.n_mtiles = (int)n_mtiles;
  p.pair_tiles = 0;
  p.total_tiles = (int)total;
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, CAUSAL, true, NW, BN, false, false, 1, true>),
                     dim3(p.total_tiles), dim3(64 * NW), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((rows + 7) / 8));
  if (out_f32)
    hipLaunchKernelGGL((prefill_split_combine_kernel<D, BF16, true>), grid, dim3(64), 0, s, a, B,
                       part_o, part_lse);
  else
    hipLaunchKernelGGL((prefill_split_combine_kernel<D, BF16, false>), grid, dim3(64), 0, s, a,
                       B, part_o, part_lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(bool bf16, bool causal, bool out_f32, const PrefillArgs& a, int B,
                          float* part_o, float* part_lse, hipStream_t s) {
  if (bf16)
    return causal ? launch_split_t<D, true, true>(a, B, part_o, part_lse, out_f32, s)
                  : launch_split_t<D, true, false>(a, B, part_o, part_lse, out_f32, s);
  return causal ? launch_split_t<D, false, true>(a, B, part_o, part_lse, out_f32, s)
                : launch_split_t<D, false, false>(a, B, part_o, part_lse, out_f32, s);
}

}  // namespace

hipError_t launch_prefill_splitkv(int D, bool bf16, bool causal, bool out_f32,
                                  const PrefillArgs& a, int B, float* part_o, float* part_lse,
                                  hipStream_t s) {
  if (D == 128) return launch_split_d<128>(bf16, causal, out_f32, a, B, part_o, part_lse, s);
  if (D == 64) return launch_split_d<64>(bf16, causal, out_f32, a, B, part_o, part_lse, s);
  return hipErrorInvalidValue;
}

namespace {
// Split-KV extend: the extend kernel in SPLIT mode (the grid of attn_extend
// times n_splits, four query heads per workgroup when the group allows it),
// then the extend combine over (row block, head) x sequence.
template <int D, bool BF16, int HPW>
hipError_t launch_ext_split_t(const PrefillArgs& a, int B, float* part_o, float* part_lse,
                              bool out_f32, hipStream_t s) {
  constexpr int NW = D == 128 ? 8 : 4;
  constexpr int BN = 64;
  constexpr int RPW = 32 * NW / HPW;
  const int64_t n_mtiles = (a.Sq + RPW - 1) / RPW;
  const int64_t total = (int64_t)B * (a.H / HPW) * n_mtiles * a.n_splits;
  const int64_t gx = (int64_t)((a.Sq + 7) / 8) * a.H;
  if (total >= ((int64_t)1 << 31) || gx >= ((int64_t)1 << 31) || B > 65535)
    return hipErrorInvalidValue;
  PrefillArgs p = a;
  p.o = part_o;
  p.lse = part_lse;
  p.n_mtiles = (int)n_mtiles;
  p.pair_tiles = 0;
  p.total_tiles = (int)total;
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, true, true, NW, BN, true, false, HPW, true>),
                     dim3(p.total_tiles), dim3(64 * NW), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)gx, (unsigned)B);
  if (out_f32)
    hipLaunchKernelGGL((extend_split_combine_kernel<D, BF16, true>), grid, dim3(64), 0, s, a,
                       part_o, part_lse);
  else
    hipLaunchKernelGGL((extend_split_combine_kernel<D, BF16, false>), grid, dim3(64), 0, s, a,
                       part_o, part_lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ext_split_d(bool bf16, bool out_f32, const PrefillArgs& a, int B,
                              float* part_o, float* part_lse, hipStream_t s) {
  const bool g4 = a.group % 4 == 0;
  if (bf16)
    return g4 ? launch_ext_split_t<D, true, 4>(a, B, part_o, part_lse, out_f32, s)
              : launch_ext_split_t<D, true, 1>(a, B, part_o, part_lse, out_f32, s);
  return g4 ? launch_ext_split_t<D, false, 4>(a, B, part_o, part_lse, out_f32, s)
            : launch_ext_split_t<D, false, 1>(a, B, part_o, part_lse, out_f32, s);
}
}  // namespace

hipError_t launch_extend_splitkv(int D, bool bf16, bool out_f32, const PrefillArgs& a, int B,
                                 float* part_o, float* part_lse, hipStream_t s) {
  if (D == 128) return launch_ext_split_d<128>(bf16, out_f32, a, B, part_o, part_lse, s);
  if (D == 64) return launch_ext_split_d<64>(bf16, out_f32, a, B, part_o, part_lse, s);
  return hipErrorInvalidValue;
}

namespace {
template <int D>
hipError_t launch_ext_d(bool bf16, bool out_f32, const PrefillArgs& a, int B, hipStream_t s) {
  constexpr int NW = D == 128 ? 8 : 4;
  constexpr int BN = 64;
  if (bf16)
    return out_f32 ? launch_g<D, true, true, true, NW, BN, true>(a, B, s)
                   : launch_g<D, true, true, false, NW, BN, true>(a, B, s);
  return out_f32 ? launch_g<D, false, true, true, NW, BN, true>(a, B, s)
                 : launch_g<D, false, true, false, NW, BN, true>(a, B, s);
}
}  // namespace

namespace {
template <int D, bool CAUSAL>
hipError_t launch_fp8_c(bool out_bf16, bool out_f32, const PrefillArgs& a, int B, hipStream_t s) {
  constexpr int NW = D == 128 ? 8 : 4;
  constexpr int BN = 64;
  if (out_f32) return launch_t<D, false, CAUSAL, true, NW, BN, false, true>(a, B, s);
  return out_bf16 ? launch_t<D, true, CAUSAL, false, NW, BN, false, true>(a, B, s)
                  : launch_t<D, false, CAUSAL, false, NW, BN, false, true>(a, B, s);
}
template <int D>
hipError_t launch_fp8_d(bool out_bf16, bool causal, bool out_f32, const PrefillArgs& a, int B,
                        hipStream_t s) {
  return causal ? launch_fp8_c<D, true>(out_bf16, out_f32, a, B, s)
                : launch_fp8_c<D, false>(out_bf16, out_f32, a, B, s);
}
}  // namespace

hipError_t launch_prefill_fp8(int D, bool out_bf16, bool causal, bool out_f32,
                              const PrefillArgs& a, int B, hipStream_t s) {
  if (D == 128) return launch_fp8_d<128>(out_bf16, causal, out_f32, a, B, s);
  if (D == 64) return launch_fp8_d<64>(out_bf16, causal, out_f32, a, B, s);
  return hipErrorInvalidValue;
}

hipError_t launch_extend(int D, bool bf16, bool out_f32, const PrefillArgs& a, int B,
                         hipStream_t s) {
  if (D == 128) return launch_ext_d<128>(bf16, out_f32, a, B, s);
  if (D == 64) return launch_ext_d<64>(bf16, out_f32, a, B, s);
  return hipErrorInvalidValue;
}

}  // namespace mi355_attn
