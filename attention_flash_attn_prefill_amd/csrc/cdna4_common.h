// Device helpers shared by the MFMA kernels (prefill.hip, decode_gqa.hip):
// vector types, the gfx950 32x32x16 MFMAs, lane-pair reductions, rounding
// conversions, the LDS chunk swizzle and vmcnt waits.  Internal; included
// inside namespace mi355_attn's anonymous namespace of each kernel file.
#pragma once

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int kBufferConfig = 0x00020000;  // raw buffer, 32-bit data format

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

// One fp32 -> fp16/bf16 bits, round to nearest even (hardware conversions).
template <bool BF16>
__device__ __forceinline__ uint16_t to_out(float f) {
  if constexpr (BF16) return __builtin_bit_cast(uint16_t, (__bf16)f);
  else return __builtin_bit_cast(uint16_t, (_Float16)f);
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

// Two fp32 -> packed bf16x2, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Packed bf16x2 -> packed fp16x2 (exact inside the fp16 normal range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// Sum / max of an int over the 64 lanes of a wave (every lane active), as a
// wave-uniform value: butterflies inside each quad and row of 16 lanes by DPP
// (quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, row_ror 8), then the four row
// results read out.
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false);
  v += __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Workgroup -> work item.  The dispatcher sends workgroup w to XCD w % 8; give
// each XCD a contiguous range of work items so one head's tiles share an L2.
// Bijective on [0, total).
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = w & 7, k = w >> 3;
  return x * q + min(x, r) + k;
}

// Workgroup -> work item for work made of `pairs` blocks of `m` items that
// read the same data (a sequence's KV head): block j runs on XCD j % 8, so a
// block's items share one L2, and every XCD gets every eighth block (with
// ragged sequences that balances the XCDs, where contiguous ranges would
// give each XCD about one sequence).  Identity unless pairs % 8 == 0.
// Bijective on [0, pairs * m).
__device__ __forceinline__ int xcd_interleave(int w, int pairs, int m) {
  if (pairs & 7) return w;
  const int x = w & 7, k = w >> 3;
  return ((k / m) * 8 + x) * m + k % m;
}

// XOR swizzle of the 16-byte chunk index within an LDS row of D halves.  For
// D = 128 (16 chunks) it swaps the two 2-bit halves of the row's low nibble:
// 16 consecutive rows read at one logical chunk (the K operand reads) land on
// 16 distinct chunk positions, and the four consecutive rows named by one
// transposing read land on distinct chunk quartets, so neither read pattern
// has bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return row & 7;
}

// XOR swizzle of the 16-byte chunk index within an LDS row of D fp8 bytes
// (8 chunks for D = 128, 4 for D = 64): the 16 lanes of a 128-bit read pass
// (rows r .. r+15 at one logical chunk) land on 16 distinct 16-byte bank
// groups.
template <int D>
__device__ __forceinline__ int swz_fp8(int row) {
  if constexpr (D == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// S^T block += K (fp8, 32 x 64) * Q^T (fp8, 64 x 32) on the gfx950 fp8 MFMA
// (e4m3fn operands, unit E8M0 scales).  Lane l holds 32 consecutive head
// dims of row / column l % 32; both operands use the same split of the 64.
__device__ __forceinline__ f32x16 mfma_qk_fp8(i32x8 a, i32x8 b, f32x16 c) {
  constexpr int kUnitScale = 127;  // E8M0 exponent code of 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kUnitScale, 0,
                                                          kUnitScale);
}

// Four e4m3fn bytes -> two packed fp16x2 (exact: every e4m3fn value is an fp16).
__device__ __forceinline__ u32x2 fp8x4_to_f16x4(uint32_t w) {
  const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// s_waitcnt that waits until at most N vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
