// Paged flash decoding for gfx950, one query per sequence, for every group
// size: the query heads that share a KV head (grouped-query and multi-query
// attention, H_kv < H; one head per KV head for multi-head attention) are
// decoded together, so each K/V row is read from HBM once for the whole
// group, and the group's queries are the N dimension of the matrix-core
// products (zero-padded to 32: the products are a small share of the time
// of this memory-bound kernel even for one query head).  Flash decoding:
// split the KV range, one partial output and log-sum-exp per piece, merge by
// log-sum-exp ("Wave February 2025 Release", FlashDecoding list; pieces sized
// to fill the GPU: "[FlyDSL] FP8 MQA logits improvements for gfx950",
// Changes / Host side).
//
// Work: a line is one (sequence, KV head, 32-query chunk of the group) and
// holds its sequence's 32-token tiles; the batch's tiles, line after line,
// are cut on the device into W equal contiguous ranges, one wave each, so
// every wave streams the same number of tiles whatever the length mix (W at
// most the resident wave count, so all ranges start at once).  A range
// writes one partial per line it touches; the combine kernel below merges a
// line's partials.  Within a range, per line:
//   * Tiles of 32 tokens (two 16-token pages).  K and V rows of a tile are
//     gathered through the page table into registers with 16-byte
//     non-temporal buffer loads (16 lanes per 256-byte row); tile t+1's loads
//     are in flight while tile t computes.  The registers then go to the
//     wave's own LDS (one stage, 16 KB: room for eight waves per CU), from
//     which the MFMA operands are read.  The bytes in flight per CU, not the
//     arithmetic, bound this kernel: staging through registers instead of
//     LDS-only double buffering lets more waves (and bytes) be resident.
//   * Each page gets its own buffer resource whose range ends at the
//     segment's last live token, so slots past it read as zero and a page
//     past the end is never touched.
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (K rows are the M dimension, the
//     group's queries the N dimension, zero-padded to 32), the online softmax
//     per query column in fp32 (base 2, lazy rescale), P rounded to fp16 and
//     O^T += V^T P^T on fp16 MFMA with V read by transposing LDS reads -- the
//     operand layouts and swizzle of the prefill kernel.
//   * Page ids are checked before any load through them: an id outside
//     [0, num_pages) poisons the segment's partial result with NaN.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace mi355_attn {
namespace {

#include "cdna4_common.h"

constexpr int PS = kDecodePageSize;  // tokens per page
constexpr int T = 2 * PS;            // tokens per tile

// P16: the partial outputs are stored in fp16 (fp16 inputs and output only:
// a partial is a convex combination of V rows, so it stays within fp16's
// range, and the output is rounded to fp16 anyway); otherwise fp32.
template <int D, bool BF16, bool P16>
__global__ __launch_bounds__(64, 2) void decode_gqa_split_kernel(DecodeArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int CPR = D / 8;           // 16-byte chunks per token row
  constexpr int LOADS = T * CPR / 64;  // 16-byte loads per lane per K (or V) tile
  static_assert(LOADS * 64 == T * CPR && LOADS % 2 == 0, "tile must split over the wave");
  constexpr int kNonTemporal = 2;      // buffer-load cache policy: streamed, read once
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[T * D];

  const int lane = threadIdx.x;
  const int li = lane & 31, hi = lane >> 5;
  const int w = blockIdx.x;  // work range
  const int lines = a.H_kv * a.qchunks;  // lines (KV head x query chunk) per sequence
  const int cap = a.max_pages * PS;      // lengths are clamped to the page table
  // Tiles of each line of sequence b.
  auto seq_tiles = [&](int b) { return (max(0, min(a.seq_lens[b], cap)) + T - 1) / T; };

  // ---- balanced work ranges.  The batch's tiles, line after line
  // (line = (b * H_kv + kv_head) * qchunks + qchunk, each line the tiles of
  // its sequence), are cut into W equal contiguous ranges, one per wave, so
  // every wave streams the same number of tiles whatever the length mix.
  // Every wave scans the lengths (K per lane per pass) for the total NT and
  // its starting sequence; wave 0 also stores NT, W and each sequence's
  // first tile for the combine.
  constexpr int K = 8;
  int c[K];
  auto load_counts = [&](int base) __attribute__((always_inline)) {
    int tot = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int bb = base + lane * K + k;
      c[k] = bb < a.B ? seq_tiles(bb) * lines : 0;
      tot += c[k];
    }
    return tot;
  };
  // Exclusive prefix over the lanes of v; *total = the sum over the wave.
  auto lane_scan = [&](int v, int* total) __attribute__((always_inline)) {
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    *total = __builtin_amdgcn_readlane(incl, 63);
    return incl - v;
  };
  int NT = 0;
  for (int base = 0; base < a.B; base += 64 * K) {
    int total;
    const int ex = lane_scan(load_counts(base), &total);
    if (w == 0) {
      int run = NT + ex;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int bb = base + lane * K + k;
        if (bb < a.B) a.meta[2 + bb] = run;
        run += c[k];
      }
    }
    NT += total;
  }
  const int W = NT == 0 ? 0 : min(a.n_splits, (NT + a.min_tiles - 1) / a.min_tiles);
  if (w == 0 && lane == 0) {
    a.meta[0] = NT;
    a.meta[1] = W;
    a.meta[2 + a.B] = NT;
  }
  if (w >= W) return;  // W <= NT: every range below W holds at least one tile
  const int s0 = (int)((int64_t)w * NT / W), s1 = (int)((int64_t)(w + 1) * NT / W);
  // The sequence holding tile s0 (the first whose tiles end past it) and its
  // first tile.
  int b0 = -1, p0 = 0;
  {
    // One pass held every length (B <= 64 K): its counts are still in c[].
    const bool one_pass = a.B <= 64 * K;
    int carry = 0;
    for (int base = 0; base < a.B && b0 < 0; base += 64 * K) {
      int total;
      int run = carry;
      if (one_pass) {
        int tot = 0;
#pragma unroll
        for (int k = 0; k < K; ++k) tot += c[k];
        run += lane_scan(tot, &total);
      } else {
        run += lane_scan(load_counts(base), &total);
      }
      int found = -1, start = 0;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (found < 0 && run + c[k] > s0) {
          found = k;
          start = run;
        }
        run += c[k];
      }
      const uint64_t m = __builtin_amdgcn_ballot_w64(found >= 0);
      if (m != 0) {
        const int src = __builtin_ctzll(m);
        b0 = base + src * K + __builtin_amdgcn_readlane(found, src);
        p0 = __builtin_amdgcn_readlane(start, src);
      }
      carry += total;
    }
  }
  if (b0 < 0) return;  // unreachable for s0 < NT

  // ---- LDS read offsets (halves): K rows li (A operand), V by transposing
  // reads (lane (g16, r, c) names 4 halves of key 8half + 4hi + r at
  // d = 32db + 16(g16 & 1) + 4c), exactly as in the prefill kernel.
  int k_rd[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) k_rd[s] = li * D + (((2 * s + hi) ^ swz<D>(li)) * 8);
  const int g16 = lane >> 4, tr_r = (lane >> 2) & 3, tr_c = lane & 3;
  int v_rd[2][D / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int key = 8 * half + 4 * hi + tr_r;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int chunk = 4 * db + 2 * (g16 & 1) + (tr_c >> 1);
      v_rd[half][db] = key * D + ((chunk ^ swz<D>(key)) * 8) + (tr_c & 1) * 4;
    }
  }
  LDS_AS uint16_t* const Ks = (LDS_AS uint16_t*)k_lds;
  LDS_AS uint16_t* const Vs = (LDS_AS uint16_t*)v_lds;

  // The lengths and the page table do not change while the kernel runs.
  // Where a wave reads one of their entries at a wave-uniform index at the
  // start of a segment, it reads through the constant address space, so the
  // read is a scalar load: a vector load there would wait (the vector memory
  // counter being shared) for the previous segment's partial stores.  The
  // per-tile page ids stay vector loads (as scalar loads they made batches of
  // 32+ tiles per range 1-2% slower).
  typedef const __attribute__((address_space(4))) int32_t* ConstI32;
  auto seq_tiles_u = [&](int b) {
    return (max(0, min(((ConstI32)a.seq_lens)[b], cap)) + T - 1) / T;
  };

  // ---- one segment: tiles [tile0, tile1) of line (b, hk, qc), written to
  // partial slot `slot` (one row per query of the chunk).
  auto segment = [&](int b, int hk, int qc, int tile0, int tile1, int slot)
                     __attribute__((always_inline)) {
    const int n = max(0, min(((ConstI32)a.seq_lens)[b], cap));
    const int t_begin = tile0 * T;
    const int t_end = min(n, tile1 * T);
    const int n_tiles = tile1 - tile0;

    // Q^T fragments (B operand): lane holds query head qc*32 + li of the group,
    // dims 16s + 8hi .. +7; columns past the group are zero.
    const int qn = qc * 32 + li;
    const bool q_ok = qn < a.group;
    const int h = hk * a.group + qn;
    u32x4 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = q_ok ? *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.H + h) * D + 16 * s + 8 * hi)
                   : (u32x4){0u, 0u, 0u, 0u};

    // ---- gather addresses.  Load i of a lane fetches tile chunk P = 64 i + lane,
    // which goes to LDS chunk P: row r = P / CPR (token r of the tile: page
    // r / 16, slot r % 16), position P % CPR, holding logical chunk
    // position ^ swz(r).
    const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
    const ConstI32 ptab_s = (ConstI32)a.page_table + (int64_t)b * a.max_pages;
    const int64_t page_elems = (int64_t)PS * a.H_kv * D;
    const uint32_t row_bytes = (uint32_t)a.H_kv * D * 2u;
    int g_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int P = 64 * i + lane;
      const int r = P / CPR, pos = P % CPR;
      g_off[i] = (((r % PS) * a.H_kv + hk) * D + ((pos ^ swz<D>(r)) * 8)) * 2;
    }
    // A page's buffer covers its first `live` slots; live = 0 covers nothing.
    auto page_rsrc = [&](const uint16_t* cache, int pg, int live) {
      const uint16_t* base = live > 0 ? cache + (int64_t)pg * page_elems : cache;
      return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(live * row_bytes),
                                               kBufferConfig);
    };

    u32x4 vreg[LOADS], kreg[LOADS];  // the next tile, in flight
    bool bad_page = false;  // wave-uniform
    // Issue the loads of the tile starting at token tb (the segment's first
    // tile: its page ids by scalar loads); false (and nothing issued) if a
    // page id lies outside the pool.
    auto issue = [&](int tb, bool first) {
      const int live0 = min(PS, t_end - tb);
      const int live1 = max(0, min(PS, t_end - tb - PS));
      const int pg0 = first ? ptab_s[tb / PS] : ptab[tb / PS];
      const int pg1 = live1 > 0 ? (first ? ptab_s[tb / PS + 1] : ptab[tb / PS + 1]) : pg0;
      if ((uint32_t)pg0 >= (uint32_t)a.num_pages || (uint32_t)pg1 >= (uint32_t)a.num_pages)
        return false;
      const auto k0 = page_rsrc(a.k_cache, pg0, live0), k1 = page_rsrc(a.k_cache, pg1, live1);
      const auto v0 = page_rsrc(a.v_cache, pg0, live0), v1 = page_rsrc(a.v_cache, pg1, live1);
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        kreg[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(i < LOADS / 2 ? k0 : k1, g_off[i], 0, kNonTemporal));
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        vreg[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(i < LOADS / 2 ? v0 : v1, g_off[i], 0, kNonTemporal));
      return true;
    };
    // Write the loaded tile to LDS (bf16 V converted to fp16 on the way).
    auto store_kv = [&](LDS_AS uint16_t* kd, LDS_AS uint16_t* vd) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        *reinterpret_cast<LDS_AS u32x4*>(kd + i * 512 + lane * 8) = kreg[i];
        u32x4 w = vreg[i];
        if constexpr (BF16) {
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = bf16x2_to_f16x2(vreg[i][j]);
        }
        *reinterpret_cast<LDS_AS u32x4*>(vd + i * 512 + lane * 8) = w;
      }
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
    float m_run = kNegInf;  // reference max (log2 units) of this lane's query column
    float l_run = 0.f;      // this lane's share of the row sum

    auto compute = [&](int tb, const LDS_AS uint16_t* ks, const LDS_AS uint16_t* vs) {
      // S^T = K Q^T (32 tokens x 32 queries).
      u32x4 kf[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) kf[s] = *reinterpret_cast<const LDS_AS u32x4*>(ks + k_rd[s]);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sc = (f32x16){};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) sc = mfma_qk<BF16>(kf[s], qf[s], sc);
      // Tokens past the segment's end.
      if (tb + T > t_end) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tb + 8 * (r >> 2) + 4 * hi + (r & 3) >= t_end) sc[r] = kNegInf;
      }
      // Row max and lazy rescale (the reference max moves only when some
      // column's max grew by more than 8 in log2 units).
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = pair_max(mx) * a.c;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
        m_run = m_new;
      }
      const float base = (m_run == kNegInf) ? 0.f : m_run;
      // P^T = exp2(S^T c - base) in fp16, and the row sum of those values.
      u32x4 pf[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * s + j], a.c, -base));
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
      // O^T += V^T P^T.
      u32x4 vf[2][D / 32];
#pragma unroll
      for (int s = 0; s < 2; ++s)
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
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma_pv(vf[s][db], pf[s], acc[db]);
    };

    // One tile per step: tile t goes registers -> LDS (the LDS writes follow
    // the previous tile's LDS reads in the wave's own order), tile t+1's loads
    // are issued, tile t is computed from LDS.
    if (!issue(t_begin, true)) bad_page = true;
    for (int t = 0; t < n_tiles && !bad_page; ++t) {
      const int tb = t_begin + t * T;
      store_kv(Ks, Vs);
      if (t + 1 < n_tiles && !issue(tb + T, false)) {
        bad_page = true;
        break;
      }
      compute(tb, Ks, Vs);
    }
    wait_vmcnt<0>();  // no load is outstanding when the segment ends

    // ---- partial result of the segment: O normalised by its row sum, and the
    // log-sum-exp in base 2.  Lane (li, hi) holds d = 32db + 8(r/4) + 4hi + r%4.
    if (!q_ok) return;
    const int64_t row = (int64_t)slot * a.rows_per_slot + li;
    // A rejected page makes the partial NaN (the key set is unknown).
    const float l_tot = pair_sum(l_run);  // > 0: the segment holds a live token
    const float inv = bad_page ? __builtin_nanf("") : 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float* v4 = reinterpret_cast<const float*>(&acc[db]) + 4 * g;
        const int d0 = 32 * db + 8 * g + 4 * hi;
        if constexpr (P16)
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.part_o) + row * D + d0) =
              (u32x2){pack_f16(v4[0] * inv, v4[1] * inv), pack_f16(v4[2] * inv, v4[3] * inv)};
        else
          *reinterpret_cast<f32x4*>(a.part_o + row * D + d0) =
              (f32x4){v4[0] * inv, v4[1] * inv, v4[2] * inv, v4[3] * inv};
      }
    if (hi == 0) a.part_lse[row] = bad_page ? __builtin_nanf("") : m_run + __log2f(l_tot);
  };

  // ---- walk the range: a segment per line it touches.
  int b = b0, pb = p0, ntb = seq_tiles_u(b0);  // ntb > 0: b0 holds tile s0
  for (int s = s0; s < s1;) {
    const int o = s - pb;
    const int j = o / ntb;  // line of sequence b
    const int t0 = o - j * ntb;
    const int t1 = min(ntb, t0 + (s1 - s));
    segment(b, j / a.qchunks, j % a.qchunks, t0, t1, w + b * lines + j);
    s += t1 - t0;
    if (s < s1 && t1 == ntb && j + 1 == lines) {  // next sequence with tiles
      pb += ntb * lines;
      do {
        ++b;
        ntb = seq_tiles_u(b);
      } while (ntb == 0);
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Merge, by log-sum-exp, the partials of the ranges that cover a (sequence,
// query head) row's line (slots w + line for the waves w whose range holds
// one of its tiles, found from NT, W and the sequence's first tile as the
// split kernel cut them).  A NaN partial (rejected page id) makes the output
// NaN; a sequence without tokens gets O = 0.
//
// Eight rows per 64-lane workgroup, eight lanes per row, each lane D/8
// consecutive outputs: a row's partial is read as 16-byte loads, the eight
// lanes of a row covering it contiguously, and up to U partials per lane are
// in flight at once (the merge is bound by load latency, not bytes).  Lanes
// first take the row's maximum log-sum-exp over the partials (each lane a
// stride-8 share, reduced over the row's lanes), then accumulate the
// partials in slot order with the same operations as a one-lane-per-output
// loop, so the result does not depend on this layout.
template <int D, bool BF16, bool OF32, bool P16>
__global__ __launch_bounds__(64) void decode_gqa_combine_kernel(DecodeArgs a) {
  constexpr int E = D / 8;                      // outputs per lane
  constexpr int EB = P16 ? 2 : 4;               // bytes per partial element
  constexpr int NV = E * EB / 16;               // 16-byte loads per lane per partial
  constexpr int U = P16 ? 16 : 8;               // partials loaded per batch
  constexpr int EPV = 16 / EB;                  // elements per 16-byte load
  static_assert(NV * 16 == E * EB, "a lane's share is whole 16-byte chunks");
  const int lane = threadIdx.x;
  const int k = lane & 7;                       // the lane's chunk of its row
  const int bh = blockIdx.x * 8 + (lane >> 3);  // the lane's (sequence, head) row
  if (bh >= a.B * a.H) return;                  // whole 8-lane groups leave together
  const int b = bh / a.H, h = bh % a.H;
  const int hk = h / a.group, qn = h % a.group;
  const int lines = a.H_kv * a.qchunks;
  const int j = hk * a.qchunks + qn / 32;  // line of sequence b
  const int NT = a.meta[0], W = a.meta[1];
  const int pb = a.meta[2 + b];
  const int ntb = (a.meta[3 + b] - pb) / lines;

  int np = 0;             // partials of the line
  int64_t row0 = 0;       // partial row of the first of them
  const int64_t stride = a.rows_per_slot;  // row of the next slot
  if (ntb > 0) {
    const int A = pb + j * ntb, Ee = A + ntb;  // the line's tiles [A, Ee)
    const int w_lo = (int)(((int64_t)(A + 1) * W - 1) / NT);
    const int w_hi = (int)(((int64_t)Ee * W - 1) / NT);
    np = w_hi - w_lo + 1;
    row0 = (int64_t)(w_lo + b * lines + j) * a.rows_per_slot + qn % 32;
  }

  // Row maximum of the partials' log-sum-exps, and whether any is NaN.
  float mx = kNegInf;
  int poisoned = 0;
  for (int s = k; s < np; s += 8) {
    const float l = a.part_lse[row0 + s * stride];
    mx = fmaxf(mx, l);
    poisoned |= __builtin_isnan(l) ? 1 : 0;
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off));
    poisoned |= __shfl_xor(poisoned, off);
  }

  float wsum = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const char* po_base = reinterpret_cast<const char*>(a.part_o) + (int64_t)k * E * EB;
  for (int s0 = 0; s0 < np; s0 += U) {
    // Loads of the batch (indices past the end repeat the last partial and
    // are not accumulated).
    float l[U];
    u32x4 p[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = row0 + min(s0 + u, np - 1) * stride;
      l[u] = a.part_lse[row];
#pragma unroll
      for (int v = 0; v < NV; ++v)
        p[u][v] = *reinterpret_cast<const u32x4*>(po_base + row * D * EB + 16 * v);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < np) {
        const float w = __builtin_amdgcn_exp2f(l[u] - mx);
        wsum += w;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          if constexpr (P16) {
            const f16x8 hv = __builtin_bit_cast(f16x8, p[u][v]);
#pragma unroll
            for (int i = 0; i < EPV; ++i)
              acc[v * EPV + i] = __builtin_fmaf(w, (float)hv[i], acc[v * EPV + i]);
          } else {
            const f32x4 fv = __builtin_bit_cast(f32x4, p[u][v]);
#pragma unroll
            for (int i = 0; i < EPV; ++i)
              acc[v * EPV + i] = __builtin_fmaf(w, fv[i], acc[v * EPV + i]);
          }
        }
      }
    }
  }
  const float inv = poisoned ? __builtin_nanf("") : (wsum > 0.f ? 1.f / wsum : 0.f);
  const int64_t o0 = (int64_t)bh * D + k * E;
  if constexpr (OF32) {
#pragma unroll
    for (int v = 0; v < E / 4; ++v)
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + o0 + 4 * v) =
          (f32x4){acc[4 * v] * inv, acc[4 * v + 1] * inv, acc[4 * v + 2] * inv,
                  acc[4 * v + 3] * inv};
  } else {
#pragma unroll
    for (int v = 0; v < E / 8; ++v) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)to_out<BF16>(acc[8 * v + 2 * i] * inv) |
               ((uint32_t)to_out<BF16>(acc[8 * v + 2 * i + 1] * inv) << 16);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + o0 + 8 * v) = w;
    }
  }
}

template <int D, bool BF16>
hipError_t launch_t(bool out_f32, const DecodeArgs& a, hipStream_t s) {
  hipError_t e;
  if (out_f32) {
    hipLaunchKernelGGL((decode_gqa_split_kernel<D, BF16, false>), dim3(a.n_splits), dim3(64), 0,
                       s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((decode_gqa_combine_kernel<D, BF16, true, false>),
                       dim3((a.B * a.H + 7) / 8), dim3(64), 0, s, a);
  } else {
    constexpr bool P16 = !BF16;
    hipLaunchKernelGGL((decode_gqa_split_kernel<D, BF16, P16>), dim3(a.n_splits), dim3(64), 0, s,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((decode_gqa_combine_kernel<D, BF16, false, P16>),
                       dim3((a.B * a.H + 7) / 8), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode_gqa(int D, bool bf16, bool out_f32, const DecodeArgs& a,
                                   hipStream_t s) {
  if (D == 128) return bf16 ? launch_t<128, true>(out_f32, a, s) : launch_t<128, false>(out_f32, a, s);
  if (D == 64) return bf16 ? launch_t<64, true>(out_f32, a, s) : launch_t<64, false>(out_f32, a, s);
  return hipErrorInvalidValue;
}

}  // namespace mi355_attn
