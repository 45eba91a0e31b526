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
// A workgroup owns 128 query rows of one (batch, head); each of its four waves
// owns 32 of them.  The wave computes the *transposed* score tile
//     S^T (64 keys x 32 queries) = K (64 x D) . Q^T (D x 32)
// with v_mfma_f32_32x32x16_{f16,bf16}: K is the A operand (read from LDS), Q^T
// is the B operand (held in VGPRs for the whole KV loop).  In the 32x32 fp32
// accumulator a lane owns one query column (lane % 32) and 16 key rows, so
//   * the row max / row sum of a query is a reduction over the lane's own
//     registers plus one v_permlane32_swap with the partner lane (lane ^ 32),
//   * the rescale factor of a query is a per-lane scalar, and
//   * exp(S^T) rounded to fp16 is already laid out as the B operand of
//     O^T (D x 32) = V^T (D x 64) . P^T (64 x 32): P never round-trips
//     through LDS.
// The MFMA sums over k in whatever order the lanes present it, so P^T's
// k-order (dictated by the accumulator layout) only has to match V^T's.  The
// V tile is therefore written to LDS transposed ([d][key]) with keys permuted
// inside each 16-key group so each lane's eight keys are contiguous
// (one 128-bit LDS read per operand).
//
// Memory path: K and V tiles (64 keys) are fetched with 128-bit coalesced
// global loads into registers while the previous tile computes, then written
// to a double-buffered LDS pair (one barrier per tile; register staging and
// double buffering per "Wave February 2025 Release", Multi-Buffering and
// EvoFormer lists; vectorised/coarsened global reads per the WAVE summary,
// lowering pipeline).  LDS rows are padded by 16 bytes so the 128-bit operand
// reads of a wave fall in distinct banks.
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

#include "kernels.h"

namespace mi355_attn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;
constexpr int NT = kPrefillThreads;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyRescale = 8.0f;  // log2 units

template <bool BF16>
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Max / sum of a value with the same value in lane ^ 32.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 -> packed fp16x2, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 h = __builtin_convertvector((f32x2){a, b}, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return bf16_bits(a) | (bf16_bits(b) << 16);
}

// Packed bf16x2 -> packed fp16x2 (exact inside the fp16 normal range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// Workgroup -> work item.  The dispatcher sends workgroup w to XCD w % 8; give
// each XCD a contiguous range of work items so one head's query tiles share
// an L2.  Bijective on [0, total).
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = w & 7, k = w >> 3;
  return x * q + min(x, r) + k;
}

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void prefill_fwd_kernel(PrefillArgs a) {
  constexpr int KSTR = D + 8;          // K tile: [BN][KSTR] halves
  constexpr int VSTR = BN + 8;         // V^T tile: [D][VSTR] halves
  constexpr int KTILE = BN * KSTR;
  constexpr int VTILE = D * VSTR;
  constexpr int KCH = BN * D / 8 / NT; // 16-byte K chunks per thread
  constexpr int VBLK = (BN / 4) * (D / 8);  // 4-key x 8-d V blocks per tile
  static_assert(KCH * NT * 8 == BN * D, "K tile must split evenly over the threads");
  static_assert(VBLK <= NT, "one V block per thread at most");
  static_assert(2 * (KTILE + VTILE) * 2 <= 80 * 1024, "two workgroups per CU must fit in LDS");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (KTILE + VTILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hi = lane >> 5;

  const int L = xcd_remap(blockIdx.x, a.total_tiles);
  const int bh = L / a.n_mtiles;
  int mt = L - bh * a.n_mtiles;
  if (CAUSAL) mt = a.n_mtiles - 1 - mt;  // heaviest query tiles first
  const int b = bh / a.H, h = bh - b * a.H;

  const uint16_t* __restrict__ qp = a.q + b * a.q_sb + h * a.q_sh;
  uint16_t* __restrict__ op = a.o + b * a.q_sb + h * a.q_sh;
  const uint16_t* __restrict__ kp = a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t* __restrict__ vp = a.v + b * a.k_sb + h * a.k_sh;

  const int m0 = mt * BM;
  const int q0 = m0 + wave * 32;
  const int qi = q0 + li;
  const bool q_ok = qi < a.Sq;

  // Q^T fragments (B operand): lane holds Q[qi][16s + 8hi .. +7].
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = q_ok ? *reinterpret_cast<const u32x4*>(qp + qi * a.q_ss + 16 * s + 8 * hi)
                 : (u32x4){0u, 0u, 0u, 0u};

  // Keys this workgroup needs: [0, kv_end).
  int kv_end = a.Skv;
  if (CAUSAL) kv_end = min(kv_end, max(0, min(m0 + BM, a.Sq) + a.causal_off));
  const int n_tiles = (kv_end + BN - 1) / BN;
  // Keys this wave needs: [0, wave_kv_end).
  const bool wave_active = q0 < a.Sq;
  const int wave_kv_end = CAUSAL ? min(a.Skv, min(q0 + 32, a.Sq) + a.causal_off) : a.Skv;

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = (f32x16){};
  float m_run = kNegInf;  // reference max (log2 units) used in the exponent
  float l_run = 0.f;      // this lane's share of the row sum

  // ---- staging: global -> registers -> LDS
  u32x4 kreg[KCH];
  u32x4 vreg[4];
  const int vkg = tid / (D / 8), vdg = tid % (D / 8);  // V block of this thread

  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + NT * r;
      const int row = c / (D / 8), col = c % (D / 8);
      kreg[r] = (kv0 + row < a.Skv)
                    ? *reinterpret_cast<const u32x4*>(kp + (kv0 + row) * a.k_ss + col * 8)
                    : (u32x4){0u, 0u, 0u, 0u};
    }
    if (tid < VBLK) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = kv0 + 4 * vkg + r;
        vreg[r] = (row < a.Skv)
                      ? *reinterpret_cast<const u32x4*>(vp + row * a.k_ss + vdg * 8)
                      : (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = lds + buf * (KTILE + VTILE);
    uint16_t* vs = ks + KTILE;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + NT * r;
      const int row = c / (D / 8), col = c % (D / 8);
      *reinterpret_cast<u32x4*>(ks + row * KSTR + col * 8) = kreg[r];
    }
    if (tid < VBLK) {
      uint32_t w[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[r][j] = BF16 ? bf16x2_to_f16x2(vreg[r][j]) : vreg[r][j];
      // keys 4*vkg .. +3 go to positions pos .. pos+3 of their 16-key group:
      // key 16s + 8a + 4h + e sits at 16s + 8h + 4a + e.
      const int pos = 16 * (vkg >> 2) + 8 * (vkg & 1) + 4 * ((vkg >> 1) & 1);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int j = d >> 1;
        u32x2 out;
        if (d & 1) {
          out[0] = (w[0][j] >> 16) | (w[1][j] & 0xffff0000u);
          out[1] = (w[2][j] >> 16) | (w[3][j] & 0xffff0000u);
        } else {
          out[0] = (w[0][j] & 0xffffu) | (w[1][j] << 16);
          out[1] = (w[2][j] & 0xffffu) | (w[3][j] << 16);
        }
        *reinterpret_cast<u32x2*>(vs + (8 * vdg + d) * VSTR + pos) = out;
      }
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * BN;
    if (t + 1 < n_tiles) load_tile(kv0 + BN);

    if (wave_active && kv0 < wave_kv_end) {
      const uint16_t* ks = lds + (t & 1) * (KTILE + VTILE);
      const uint16_t* vs = ks + KTILE;

      // S^T = K Q^T : two 32-key blocks.
      f32x16 sacc[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        sacc[jb] = (f32x16){};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const u32x4 kf =
              *reinterpret_cast<const u32x4*>(ks + (32 * jb + li) * KSTR + 16 * s + 8 * hi);
          sacc[jb] = mfma_qk<BF16>(kf, qf[s], sacc[jb]);
        }
      }

      // Mask keys past the sequence end and (causal) above the diagonal.
      const bool need_mask =
          (kv0 + BN > a.Skv) || (CAUSAL && kv0 + BN - 1 > q0 + a.causal_off);
      if (need_mask) {
        const int lim = CAUSAL ? min(a.Skv - 1, qi + a.causal_off) : a.Skv - 1;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * jb + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key > lim) sacc[jb][r] = kNegInf;
          }
      }

      // Row max over the 64 keys (own 32 values + the partner lane's 32).
      float mx = kNegInf;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[jb][r]);
      mx = pair_max(mx) * a.c;

      // Lazy rescale: move the reference max only when a row's max grew by > 8.
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
        m_run = m_new;
      }
      const float base = (m_run == kNegInf) ? 0.f : m_run;

      // P^T = exp2(S^T * c - base) in fp16: B operand fragments for P.V.
      u32x4 pf[BN / 16];
#pragma unroll
      for (int s = 0; s < BN / 16; ++s) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + j], a.c, -base));
        // Keep the pairs as f16x2 values: clang lowers a bit-cast of an
        // ext-vector *element* (pf[s][j]) as a read of element 0.
        f16x2 h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = __builtin_convertvector((f32x2){e[2 * j], e[2 * j + 1]}, f16x2);
        pf[s] = (u32x4){__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                        __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])};
        // row sum of the rounded P (the values P.V actually uses)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          l_run = __builtin_amdgcn_fdot2(h[j], (f16x2){(_Float16)1.0f, (_Float16)1.0f}, l_run,
                                         false);
      }

      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int s = 0; s < BN / 16; ++s) {
          const u32x4 vf =
              *reinterpret_cast<const u32x4*>(vs + (32 * db + li) * VSTR + 16 * s + 8 * hi);
          acc[db] = mfma_pv(vf, pf[s], acc[db]);
        }
    }

    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l.  Lane owns query qi and, in block db, the four
  // consecutive d = 32db + 8g + 4hi .. +3 for g = 0..3.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* orow = op + qi * a.q_ss;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float* v4 = reinterpret_cast<const float*>(&acc[db]) + 4 * g;
        u32x2 out;
        if constexpr (BF16) {
          out[0] = pack_bf16(v4[0] * inv, v4[1] * inv);
          out[1] = pack_bf16(v4[2] * inv, v4[3] * inv);
        } else {
          out[0] = pack_f16(v4[0] * inv, v4[1] * inv);
          out[1] = pack_f16(v4[2] * inv, v4[3] * inv);
        }
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * hi) = out;
      }
  }
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_fwd_kernel<D, BF16, CAUSAL>), dim3(a.total_tiles), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_c(bool causal, const PrefillArgs& a, hipStream_t s) {
  return causal ? launch_t<D, BF16, true>(a, s) : launch_t<D, BF16, false>(a, s);
}

template <int D>
hipError_t launch_d(bool bf16, bool causal, const PrefillArgs& a, hipStream_t s) {
  return bf16 ? launch_c<D, true>(causal, a, s) : launch_c<D, false>(causal, a, s);
}

}  // namespace

hipError_t launch_prefill(int D, bool bf16, bool causal, const PrefillArgs& a, hipStream_t s) {
  if (D == 128) return launch_d<128>(bf16, causal, a, s);
  if (D == 64) return launch_d<64>(bf16, causal, a, s);
  return hipErrorInvalidValue;
}

}  // namespace mi355_attn
