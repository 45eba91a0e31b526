// Backward of flash attention for gfx950 (backward flash attention is a
// roadmap item of "Wave February 2025 Release"; the gradients are the chain
// rule through O = softmax(scale Q K^T + M) V, recomputing P from the
// forward's per-row log-sum-exp as flash attention does):
//
//   P = exp(scale S - LSE),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - delta),   delta_i = rowsum(dO_i * O_i),
//   dQ = scale dS K,         dK = scale dS^T Q.
//
// Three kernels:
//   * delta: per query row, rowsum(dO * O) and -LSE log2(e) in fp32 (one
//     16-byte load per lane per tensor).
//   * dK/dV: one workgroup per (batch, KV head, 128 keys), four pairs of
//     waves, a pair per 32 keys.  The pair keeps its keys' K (one wave) and V
//     (the other) as MFMA operands and dV^T, dK^T as fp32 accumulators in
//     registers for the whole pass; tiles of 64 queries of every query head
//     that shares the KV head stream through LDS (Q, dO by DMA,
//     double-buffered, plus their LSE and delta), so grouped heads sum into
//     dK, dV without atomics.  S = Q K^T and dP = dO V^T come out with a lane
//     per key and rows of queries, which is the B-operand layout of
//     dV^T += dO^T P and dK^T += Q^T dS, whose A operands (dO^T, Q^T) are read
//     by transposing LDS reads; P passes from one wave of the pair to the
//     other through LDS.
//   * dQ: one workgroup per (batch, head, 256 queries), eight waves of 32
//     queries (the forward kernel's shape): Q and dO stay as operands, tiles
//     of 64 keys stream through LDS (used as two 32-key halves), S^T = K Q^T
//     and dP^T = V dO^T give a lane per query, and dQ^T += K^T dS^T with K^T
//     by transposing reads.
// Recomputing S and dP in both kernels costs two extra products over the
// five of the algorithm but needs no fp32 atomics: the gradients are
// deterministic.  The operand layouts, swizzle and transposing-read offsets
// are the prefill kernel's.
//
// Precision: S and dP accumulate in fp32; P and dS are rounded to the input
// type (fp16 or bf16) as MFMA operands; dO stays in its own type.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace mi355_attn {
namespace {

#include "cdna4_common.h"

constexpr float kLog2e = 1.4426950408889634f;

template <bool BF16>
__device__ __forceinline__ float lo_f32(uint32_t w) {
  if constexpr (BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(f16x2, w)[0];
}
template <bool BF16>
__device__ __forceinline__ float hi_f32(uint32_t w) {
  if constexpr (BF16) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(f16x2, w)[1];
}
// Two fp32 -> packed pair in the input type (round to nearest even).
template <bool BF16>
__device__ __forceinline__ uint32_t pack_in(float x, float y) {
  if constexpr (BF16) return pack_bf16(x, y);
  else return pack_f16(x, y);
}

// -LSE in log2 units, so that P = exp2(S c + nl2); a row with no visible key
// (LSE = -inf) gets -inf, hence P = 0.
__device__ __forceinline__ float nl2_of(float lse) {
  return lse > kNegInf ? -lse * kLog2e : kNegInf;
}

// ------------------------------------------------------------------ delta
// Per query row: delta = rowsum(dO * O) and nl2 = -LSE log2(e).

template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BackwardArgs a) {
  constexpr int G = D / 8;        // lanes per row
  constexpr int RPB = 256 / G;    // rows per workgroup
  const int t = threadIdx.x;
  const int gl = t % G;
  const int64_t rows = (int64_t)a.B * a.H * a.Sq;
  const int64_t row = (int64_t)blockIdx.x * RPB + t / G;  // (b, h, i) flattened
  float acc = 0.f;
  if (row < rows) {
    const int i = (int)(row % a.Sq);
    const int64_t bh = row / a.Sq;
    const int h = (int)(bh % a.H), b = (int)(bh / a.H);
    const int64_t off = b * a.q_sb + h * a.q_sh + (int64_t)i * a.q_ss + gl * 8;
    const u32x4 o4 = *reinterpret_cast<const u32x4*>(a.o + off);
    const u32x4 d4 = *reinterpret_cast<const u32x4*>(a.dO + off);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc += lo_f32<BF16>(o4[j]) * lo_f32<BF16>(d4[j]) + hi_f32<BF16>(o4[j]) * hi_f32<BF16>(d4[j]);
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (gl == 0 && row < rows) {
    a.delta[row] = acc;
    a.nl2[row] = nl2_of(a.lse[row]);
  }
}

// Store 4 consecutive values of a gradient row (dtype or fp32).
template <bool BF16, bool OF32>
__device__ __forceinline__ void store4(void* base, int64_t off, const float* v, float f) {
  if constexpr (OF32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) =
        (f32x4){v[0] * f, v[1] * f, v[2] * f, v[3] * f};
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + off) =
        (u32x2){pack_in<BF16>(v[0] * f, v[1] * f), pack_in<BF16>(v[2] * f, v[3] * f)};
  }
}

// ------------------------------------------------------------------- dK/dV

// One workgroup per (batch, KV head, 128 keys): four pairs of waves, a pair
// per 32 keys.  In a pair the P-wave (waves 0-3) holds the keys' K as MFMA
// operand and dV^T as accumulator, the D-wave (waves 4-7) holds V and dK^T;
// both walk the same 64-query tiles of Q and dO (every query head of the
// group) staged in LDS.  Per tile: the P-wave forms S = Q K^T and
// P = exp2(S c + nl2) (fp32) while the D-wave forms dP = dO V^T; P goes to
// LDS; after a barrier the P-wave accumulates dV^T += dO^T P and the D-wave
// reads P, forms dS = P (dP - delta) and accumulates dK^T += Q^T dS.  Each
// wave issues half of the tile's MFMAs, and two waves share each SIMD.
template <int D, bool BF16, bool CAUSAL, bool OF32>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BackwardArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 8;                 // four pairs of waves
  constexpr int NT = 64 * NW;
  constexpr int BK = 32 * (NW / 2);     // keys per workgroup
  constexpr int BQ = 64;                // queries per streamed tile
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int LOADS = BQ * CPR / NT;  // chunk loads per thread per Q (or dO) tile
  static_assert(LOADS * NT == BQ * CPR, "tile must split evenly over the threads");
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds0[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds1[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t do_lds0[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t do_lds1[BQ * D];
  // nl2 (floats 0..63) and delta (64..127) of a tile's rows.
  __shared__ __attribute__((aligned(512))) float rs_lds0[2 * BQ];
  __shared__ __attribute__((aligned(512))) float rs_lds1[2 * BQ];
  // P of a tile, P-wave -> D-wave: [pair][block][4 quads][64 lanes] x f32x4.
  __shared__ __attribute__((aligned(1024))) f32x4 p_lds[(NW / 2) * (BQ / 32) * 4 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave / (NW / 2);  // 0: P-wave (K, dV), 1: D-wave (V, dK); wave-uniform
  const int kw = wave % (NW / 2);    // the pair
  const int li = lane & 31, hi = lane >> 5;

  const int n_kb = a.n_tiles;
  int L = xcd_remap(blockIdx.x, a.total);
  const int kb = L % n_kb;
  L /= n_kb;
  const int hk = L % a.H_kv, b = L / a.H_kv;

  const int j0 = kb * BK;
  const int jw = j0 + 32 * kw;  // the pair's first key
  const int jl = jw + li;       // this lane's key
  const bool k_ok = jl < a.Skv;
  const int64_t kv_base = b * a.k_sb + hk * a.k_sh;

  // K^T (P-wave) or V^T (D-wave) fragments (B operands): lane holds row jl,
  // dims 16s + 8hi .. +7.
  const uint16_t* const kv_src = role == 0 ? a.k : a.v;
  u32x4 kvf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int64_t off = kv_base + (int64_t)jl * a.k_ss + 16 * s + 8 * hi;
    kvf[s] = k_ok ? *reinterpret_cast<const u32x4*>(kv_src + off) : (u32x4){0u, 0u, 0u, 0u};
  }

  // Query tiles: every query head of the group, from the first tile with a
  // query that sees one of this workgroup's keys (causal: i >= j - off).
  const int q_first = CAUSAL ? max(0, j0 - a.causal_off) : 0;
  const int qt0 = q_first / BQ;
  const int n_qt = (a.Sq + BQ - 1) / BQ - qt0;  // per head (may be <= 0)
  const int steps = n_qt > 0 ? a.group * n_qt : 0;

  // ---- staging (loop invariant pieces).
  int g_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int chunk = (wave * LOADS + i) * 64 + lane;
    const int row = chunk / CPR, pos = chunk % CPR;
    g_off[i] = (row * a.q_ss + ((pos ^ swz<D>(row)) * 8)) * 2;
  }
  const uint32_t row_bytes = (uint32_t)a.q_ss * 2u;
  // A step's position: query head h (of the group), query tile t.  One query
  // head per KV head: the tiles in order.  Several (grouped heads): the
  // tiles from the last down with the group's heads innermost, so all the
  // resident workgroups of a KV head read the same Q/dO tile at about the
  // same time (causal: they all start at the last tile, whatever their first
  // one) and the group's larger Q/dO stream comes from HBM about once per
  // XCD.  In order, each head a workgroup finishes puts it further out of
  // step with the others and their shared tiles drop out of L2 in between.
  struct Pos {
    int h, t;
  };
  const int qt_end = qt0 + n_qt;
  const int h_first = hk * a.group, h_end = h_first + a.group;
  const bool grouped = a.group > 1;  // uniform
  auto advance = [&](Pos p) __attribute__((always_inline)) {
    if (grouped) return p.h + 1 < h_end ? Pos{p.h + 1, p.t} : Pos{h_first, p.t - 1};
    return p.t + 1 < qt_end ? Pos{p.h, p.t + 1} : Pos{p.h + 1, qt0};
  };
  auto issue = [&](Pos p, LDS_AS uint16_t* qd, LDS_AS uint16_t* dd, LDS_AS float* rd) __attribute__((always_inline)) {
    const int h = p.h, i0 = p.t * BQ;
    const int64_t base = b * a.q_sb + h * a.q_sh + (int64_t)i0 * a.q_ss;
    const uint32_t rows = (uint32_t)max(0, a.Sq - i0);
    const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + base), (short)0,
                                                      (int)(rows * row_bytes), kBufferConfig);
    const auto rdo = __builtin_amdgcn_make_buffer_rsrc((void*)(a.dO + base), (short)0,
                                                       (int)(rows * row_bytes), kBufferConfig);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (LDS_AS void*)(qd + (wave * LOADS + i) * 512),
                                               16, g_off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rdo, (LDS_AS void*)(dd + (wave * LOADS + i) * 512),
                                               16, g_off[i], 0, 0, 0);
    }
    if (wave == 0) {  // 64 rows of nl2 and of delta: one float per lane (the
      // rows start at any float, so no wider access); rows past Sq read 0.
      const int64_t rbase = ((int64_t)b * a.H + h) * a.Sq + i0;
      const int nb = (int)(min((uint32_t)BQ, rows) * 4u);
      const auto rl = __builtin_amdgcn_make_buffer_rsrc((void*)(a.nl2 + rbase), (short)0, nb,
                                                        kBufferConfig);
      const auto rt = __builtin_amdgcn_make_buffer_rsrc((void*)(a.delta + rbase), (short)0, nb,
                                                        kBufferConfig);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (LDS_AS void*)rd, 4, lane * 4, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (LDS_AS void*)(rd + BQ), 4, lane * 4, 0, 0, 0);
    }
  };

  // LDS read offsets (halves): rows 32ib + li at logical chunk 2s + hi, and
  // the transposing reads (rows 16s2 + 8half + 4hi + r, d = 32db + ...).
  int r_rd[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) r_rd[s] = li * D + (((2 * s + hi) ^ swz<D>(li)) * 8);
  const int g16 = lane >> 4, tr_r = (lane >> 2) & 3, tr_c = lane & 3;
  int t_rd[2][D / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int key = 8 * half + 4 * hi + tr_r;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int chunk = 4 * db + 2 * (g16 & 1) + (tr_c >> 1);
      t_rd[half][db] = key * D + ((chunk ^ swz<D>(key)) * 8) + (tr_c & 1) * 4;
    }
  }
  auto tr_frag = [&](const LDS_AS uint16_t* base, int half0_off, int db) __attribute__((always_inline)) {
    const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (LDS_AS fp16x4_t*)(base + half0_off + t_rd[0][db]));
    const fp16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (LDS_AS fp16x4_t*)(base + half0_off + t_rd[1][db]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, up);
    return (u32x4){l2[0], l2[1], h2[0], h2[1]};
  };
  // This lane's quad q of block ib in the pair's P exchange.
  LDS_AS f32x4* const xch = (LDS_AS f32x4*)p_lds + kw * (BQ / 32) * 4 * 64 + lane;

  f32x16 acc[D / 32];  // dV^T (P-wave) or dK^T (D-wave)
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};

  // Rows past Sq read Q, dO, LSE and delta as zeros (buffer bounds), so P = 1
  // and dS = 0 there, and they add exactly 0 to dV = P^T dO and dK = dS^T Q;
  // keys past Skv are never stored; a row that sees no key has LSE = -inf and
  // P = 0.  Only the causal diagonal needs a mask.
  //
  // Before the barrier: the P-wave's S, P (written to LDS and packed as the
  // dV operand), or the D-wave's dP; lane value r of block ib is query row
  // i0 + 32ib + 8(r/4) + 4hi + r%4, key jl.  keep[ib] carries across the
  // barrier the D-wave's dP, or in its first 8 words the P-wave's packed P
  // (the roles are exclusive, so they share the registers).
  f32x16 keep[BQ / 32];
  auto phase1 = [&](auto role_c, int i0, const LDS_AS uint16_t* qs, const LDS_AS uint16_t* ds,
                    const LDS_AS float* rs) __attribute__((always_inline)) {
    if constexpr (decltype(role_c)::value == 0) {
      // Causal mask: visible iff dq >= -(32ib + 8(r/4) + r%4).
      const int dq = i0 + 4 * hi - (jl - a.causal_off);
#pragma unroll
      for (int ib = 0; ib < BQ / 32; ++ib) {
        u32x4 fq[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          fq[s] = *reinterpret_cast<const LDS_AS u32x4*>(qs + 32 * ib * D + r_rd[s]);
        f32x16 sc = (f32x16){};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) sc = mfma_qk<BF16>(fq[s], kvf[s], sc);
        float p[16];
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const f32x4 l4 = *reinterpret_cast<const LDS_AS f32x4*>(rs + 32 * ib + 8 * grp + 4 * hi);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p[4 * grp + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * grp + e], a.c, l4[e]));
        }
        // The mask only on blocks that cross the diagonal of the pair's keys
        // (a wave-uniform branch).
        if (CAUSAL && jw + 31 > i0 + 32 * ib + a.causal_off) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            p[r] = dq >= -(32 * ib + 8 * (r >> 2) + (r & 3)) ? p[r] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xch[(ib * 4 + q) * 64] = (f32x4){p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]};
        // Values r = 8 s2 + j go to operand s2, slot j (the forward's P
        // layout): word w of keep holds values 2w, 2w+1.
#pragma unroll
        for (int w = 0; w < 8; ++w)
          keep[ib][w] = __uint_as_float(pack_in<BF16>(p[2 * w], p[2 * w + 1]));
      }
    } else {
#pragma unroll
      for (int ib = 0; ib < BQ / 32; ++ib) {
        u32x4 fd[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          fd[s] = *reinterpret_cast<const LDS_AS u32x4*>(ds + 32 * ib * D + r_rd[s]);
        keep[ib] = (f32x16){};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) keep[ib] = mfma_qk<BF16>(fd[s], kvf[s], keep[ib]);
      }
    }
  };
  // After the barrier: dV^T += dO^T P (P-wave), or dS = P (dP - delta) and
  // dK^T += Q^T dS (D-wave); contraction over the block's rows.
  auto phase2 = [&](auto role_c, const LDS_AS uint16_t* qs, const LDS_AS uint16_t* ds,
                    const LDS_AS float* rs) __attribute__((always_inline)) {
    if constexpr (decltype(role_c)::value == 0) {
#pragma unroll
      for (int ib = 0; ib < BQ / 32; ++ib)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 td[D / 32];
#pragma unroll
          for (int db = 0; db < D / 32; ++db) td[db] = tr_frag(ds, (32 * ib + 16 * s2) * D, db);
          const u32x4 pf = {__float_as_uint(keep[ib][4 * s2]), __float_as_uint(keep[ib][4 * s2 + 1]),
                            __float_as_uint(keep[ib][4 * s2 + 2]), __float_as_uint(keep[ib][4 * s2 + 3])};
#pragma unroll
          for (int db = 0; db < D / 32; ++db) acc[db] = mfma_qk<BF16>(td[db], pf, acc[db]);
        }
    } else {
#pragma unroll
      for (int ib = 0; ib < BQ / 32; ++ib) {
        u32x4 sf[2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 p4 = xch[(ib * 4 + q) * 64];
          const f32x4 t4 = *reinterpret_cast<const LDS_AS f32x4*>(rs + BQ + 32 * ib + 8 * q + 4 * hi);
          // values r = 4q .. 4q+3: operand q / 2, slots 4(q % 2) ..
          sf[q >> 1][2 * (q & 1)] = pack_in<BF16>(p4[0] * (keep[ib][4 * q] - t4[0]),
                                                   p4[1] * (keep[ib][4 * q + 1] - t4[1]));
          sf[q >> 1][2 * (q & 1) + 1] = pack_in<BF16>(p4[2] * (keep[ib][4 * q + 2] - t4[2]),
                                                       p4[3] * (keep[ib][4 * q + 3] - t4[3]));
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 tq[D / 32];
#pragma unroll
          for (int db = 0; db < D / 32; ++db) tq[db] = tr_frag(qs, (32 * ib + 16 * s2) * D, db);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) acc[db] = mfma_qk<BF16>(tq[db], sf[s2], acc[db]);
        }
      }
    }
  };

  LDS_AS uint16_t* const Qs[2] = {(LDS_AS uint16_t*)q_lds0, (LDS_AS uint16_t*)q_lds1};
  LDS_AS uint16_t* const Ds[2] = {(LDS_AS uint16_t*)do_lds0, (LDS_AS uint16_t*)do_lds1};
  LDS_AS float* const Rs[2] = {(LDS_AS float*)rs_lds0, (LDS_AS float*)rs_lds1};
  // Two barriers per tile: the first makes the tile's DMA visible and frees
  // the other buffers (and the P exchange) from the previous tile; the
  // second hands P from the P-waves to the D-waves.  Each role runs its own
  // copy of the loop (same trip count, same barriers), so the registers of
  // one role's work are not held across the other's.
  auto run = [&](auto role_c) __attribute__((always_inline)) {
    Pos cur{h_first, grouped ? qt_end - 1 : qt0};
    Pos nxt = advance(cur);
    if (steps > 0) issue(cur, Qs[0], Ds[0], Rs[0]);
    auto iteration = [&](int u, auto par) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      wait_vmcnt<0>();
      __syncthreads();
      if (u + 1 < steps) issue(nxt, Qs[P ^ 1], Ds[P ^ 1], Rs[P ^ 1]);
      const int i0 = cur.t * BQ;
      // Skip a tile whose queries all precede the pair's keys (pair-uniform).
      const bool active = !CAUSAL || i0 + BQ - 1 >= jw - a.causal_off;
      if (active) phase1(role_c, i0, Qs[P], Ds[P], Rs[P]);
      __syncthreads();
      if (active) phase2(role_c, Qs[P], Ds[P], Rs[P]);
      cur = nxt;
      nxt = advance(nxt);
    };
    for (int u = 0; u < steps; u += 2) {
      iteration(u, std::integral_constant<int, 0>{});
      if (u + 1 < steps) iteration(u + 1, std::integral_constant<int, 1>{});
    }
  };
  if (role == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});

  // dV = P^T dO (P-wave), dK = scale dS^T Q (D-wave); lane holds row jl,
  // d = 32db + 8g + 4hi .. +3.
  if (k_ok) {
    const int64_t row = kv_base + (int64_t)jl * a.k_ss;
    void* const dst = role == 0 ? a.dv : a.dk;
    const float f = role == 0 ? 1.f : a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<BF16, OF32>(dst, row + 32 * db + 8 * g + 4 * hi,
                           reinterpret_cast<const float*>(&acc[db]) + 4 * g, f);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------- dQ

template <int D, bool BF16, bool CAUSAL, bool OF32, int NW>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(BackwardArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NW;           // queries per workgroup
  constexpr int BN = 64;                // keys per streamed tile (two 32-key halves)
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / NT;
  static_assert(LOADS * NT == BN * CPR, "tile must split evenly over the threads");
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hi = lane >> 5;

  int L = xcd_remap(blockIdx.x, a.total);
  const int g = L % a.group;
  L /= a.group;
  int mt = L % a.n_tiles;
  L /= a.n_tiles;
  if (CAUSAL) mt = a.n_tiles - 1 - mt;  // heaviest first
  const int hk = L % a.H_kv, b = L / a.H_kv;
  const int h = hk * a.group + g;

  const int m0 = mt * BM;
  const int q0 = m0 + 32 * wave;
  const int qi = q0 + li;
  const bool q_ok = qi < a.Sq;
  const int64_t q_row = b * a.q_sb + h * a.q_sh + (int64_t)qi * a.q_ss;

  // Q^T and dO^T fragments (B operands): lane holds row qi, dims 16s + 8hi ...
  u32x4 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = q_ok ? *reinterpret_cast<const u32x4*>(a.q + q_row + 16 * s + 8 * hi)
                 : (u32x4){0u, 0u, 0u, 0u};
    df[s] = q_ok ? *reinterpret_cast<const u32x4*>(a.dO + q_row + 16 * s + 8 * hi)
                 : (u32x4){0u, 0u, 0u, 0u};
  }
  const int64_t rid = ((int64_t)b * a.H + h) * a.Sq + qi;
  const float nl2 = q_ok ? a.nl2[rid] : kNegInf;
  const float delta = q_ok ? a.delta[rid] : 0.f;

  int kv_end = a.Skv;
  if (CAUSAL) kv_end = min(kv_end, max(0, min(m0 + BM, a.Sq) + a.causal_off));
  const int n_kt = (kv_end + BN - 1) / BN;
  const bool wave_active = q0 < a.Sq;
  const int wave_kv_end = CAUSAL ? min(a.Skv, min(q0 + 32, a.Sq) + a.causal_off) : a.Skv;

  const int64_t kv_base = b * a.k_sb + hk * a.k_sh;
  int g_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int chunk = (wave * LOADS + i) * 64 + lane;
    const int row = chunk / CPR, pos = chunk % CPR;
    g_off[i] = (row * a.k_ss + ((pos ^ swz<D>(row)) * 8)) * 2;
  }
  const uint32_t row_bytes = (uint32_t)a.k_ss * 2u;
  auto issue = [&](int t, LDS_AS uint16_t* kd, LDS_AS uint16_t* vd) __attribute__((always_inline)) {
    const int kv0 = t * BN;
    const uint32_t rows = (uint32_t)max(0, a.Skv - kv0);
    const int64_t base = kv_base + (int64_t)kv0 * a.k_ss;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + base), (short)0,
                                                      (int)(rows * row_bytes), kBufferConfig);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + base), (short)0,
                                                      (int)(rows * row_bytes), kBufferConfig);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS_AS void*)(kd + (wave * LOADS + i) * 512),
                                               16, g_off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS_AS void*)(vd + (wave * LOADS + i) * 512),
                                               16, g_off[i], 0, 0, 0);
    }
  };

  int r_rd[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) r_rd[s] = li * D + (((2 * s + hi) ^ swz<D>(li)) * 8);
  const int g16 = lane >> 4, tr_r = (lane >> 2) & 3, tr_c = lane & 3;
  int t_rd[2][D / 32];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int key = 8 * half + 4 * hi + tr_r;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int chunk = 4 * db + 2 * (g16 & 1) + (tr_c >> 1);
      t_rd[half][db] = key * D + ((chunk ^ swz<D>(key)) * 8) + (tr_c & 1) * 4;
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};

  auto compute_half = [&](int kv0, const LDS_AS uint16_t* ks, const LDS_AS uint16_t* vs) __attribute__((always_inline)) {
    // S^T = K Q^T and dP^T = V dO^T: 32 keys (rows) x 32 queries (lane).
    u32x4 fk[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) fk[s] = *reinterpret_cast<const LDS_AS u32x4*>(ks + r_rd[s]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sc = (f32x16){};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) sc = mfma_qk<BF16>(fk[s], qf[s], sc);
    u32x4 fv[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) fv[s] = *reinterpret_cast<const LDS_AS u32x4*>(vs + r_rd[s]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 dp = (f32x16){};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) dp = mfma_qk<BF16>(fv[s], df[s], dp);
    // dS^T = P^T (dP^T - delta); value r is key kv0 + 8(r/4) + 4hi + r%4.
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], a.c, nl2));
    // Keys past the end or (causal) above the diagonal, only in the halves
    // that have any: a wave-uniform branch around the whole pass, so the
    // other halves carry no per-element compares and selects (the fence has
    // a side effect, which keeps the compiler from turning the branch into
    // selects executed on every half).
    const bool need_mask = (kv0 + 32 > a.Skv) || (CAUSAL && kv0 + 31 > q0 + a.causal_off);
    if (need_mask) {
      __builtin_amdgcn_sched_barrier(0);
      const int lim = CAUSAL ? min(a.Skv - 1, qi + a.causal_off) : a.Skv - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kv0 + 8 * (r >> 2) + 4 * hi + (r & 3) > lim) p[r] = 0.f;
    }
    u32x4 sf[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float d[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) d[j] = p[8 * s2 + j] * (dp[8 * s2 + j] - delta);
#pragma unroll
      for (int w = 0; w < 4; ++w) sf[s2][w] = pack_in<BF16>(d[2 * w], d[2 * w + 1]);
    }
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 tk[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const fp16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (LDS_AS fp16x4_t*)(ks + 16 * s2 * D + t_rd[0][db]));
        const fp16x4_t up = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (LDS_AS fp16x4_t*)(ks + 16 * s2 * D + t_rd[1][db]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, up);
        tk[db] = (u32x4){l2[0], l2[1], h2[0], h2[1]};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma_qk<BF16>(tk[db], sf[s2], acc[db]);
    }
  };
  // A 64-key tile as two 32-key halves (one barrier per 64 keys); the second
  // half only if the wave sees one of its keys (wave-uniform).
  auto compute = [&](int t, const LDS_AS uint16_t* ks, const LDS_AS uint16_t* vs) __attribute__((always_inline)) {
    compute_half(t * BN, ks, vs);
    if (t * BN + 32 < wave_kv_end) compute_half(t * BN + 32, ks + 32 * D, vs + 32 * D);
  };

  LDS_AS uint16_t* const Ks[2] = {(LDS_AS uint16_t*)k_lds0, (LDS_AS uint16_t*)k_lds1};
  LDS_AS uint16_t* const Vs[2] = {(LDS_AS uint16_t*)v_lds0, (LDS_AS uint16_t*)v_lds1};
  if (n_kt > 0) issue(0, Ks[0], Vs[0]);
  auto iteration = [&](int t, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < n_kt) issue(t + 1, Ks[P ^ 1], Vs[P ^ 1]);
    if (wave_active && t * BN < wave_kv_end) compute(t, Ks[P], Vs[P]);
  };
  for (int t = 0; t < n_kt; t += 2) {
    iteration(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_kt) iteration(t + 1, std::integral_constant<int, 1>{});
  }

  if (q_ok) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        store4<BF16, OF32>(a.dq, q_row + 32 * db + 8 * gg + 4 * hi,
                           reinterpret_cast<const float*>(&acc[db]) + 4 * gg, a.scale);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool BF16, bool CAUSAL, bool OF32>
hipError_t launch_t(BackwardArgs a, hipStream_t s) {
  constexpr int NWQ = D == 128 ? 8 : 4;
  {
    constexpr int RPB = 256 / (D / 8);
    const int64_t rows = (int64_t)a.B * a.H * a.Sq;
    if (rows > 0)
      hipLaunchKernelGGL((bwd_delta_kernel<D, BF16>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                         dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BackwardArgs ak = a;
  ak.n_tiles = (a.Skv + 127) / 128;
  ak.total = a.B * a.H_kv * ak.n_tiles;
  if (ak.total > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BF16, CAUSAL, OF32>), dim3(ak.total), dim3(512), 0, s,
                       ak);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  BackwardArgs aq = a;
  aq.n_tiles = (a.Sq + 32 * NWQ - 1) / (32 * NWQ);
  aq.total = a.B * a.H * aq.n_tiles;
  if (aq.total > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, CAUSAL, OF32, NWQ>), dim3(aq.total),
                       dim3(64 * NWQ), 0, s, aq);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_c(bool causal, bool out_f32, const BackwardArgs& a, hipStream_t s) {
  if (causal) return out_f32 ? launch_t<D, BF16, true, true>(a, s) : launch_t<D, BF16, true, false>(a, s);
  return out_f32 ? launch_t<D, BF16, false, true>(a, s) : launch_t<D, BF16, false, false>(a, s);
}

}  // namespace

hipError_t launch_prefill_backward(int D, bool bf16, bool causal, bool out_f32,
                                   const BackwardArgs& a, hipStream_t s) {
  if (D == 128) return bf16 ? launch_c<128, true>(causal, out_f32, a, s)
                            : launch_c<128, false>(causal, out_f32, a, s);
  if (D == 64) return bf16 ? launch_c<64, true>(causal, out_f32, a, s)
                           : launch_c<64, false>(causal, out_f32, a, s);
  return hipErrorInvalidValue;
}

}  // namespace mi355_attn
