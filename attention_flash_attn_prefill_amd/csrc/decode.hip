// Split-KV paged flash decoding for gfx950: one query per sequence against a
// paged KV cache (flash decoding with a page table: "Wave February 2025
// Release", FlashDecoding list; splitting the KV range over extra workgroups
// and merging the partial results: "[FlyDSL] FP8 MQA logits improvements for
// gfx950", Summary and Changes / Host side).
//
// The work is HBM-bound (about one flop per byte), so the design is about the
// memory path, not the matrix cores:
//
//   * Cache layout [num_pages][16 tokens][H][D]: one token's K row for a head
//     is D*2 contiguous bytes, and a page holds 16 tokens of every head.
//   * A wave owns one (sequence, head, split).  Its lanes form groups of D/8
//     lanes; each group reads one token's K (and V) row with 128-bit loads, so
//     a wave-wide load instruction covers 4 (D = 128) or 8 (D = 64) tokens.
//   * The wave walks its split four pages (64 tokens) at a time and issues all
//     K and V loads of the batch before any arithmetic: 32 128-bit loads in
//     flight per lane (D = 128).  The loads are non-temporal: every cache byte
//     is read once per call, so it should not displace anything in L2/MALL.
//     Page ids are wave-uniform (scalar loads) and page bases use 64-bit
//     offsets (an 8 GiB pool exceeds 2^32 elements).
//   * Scores are fp32 dot products (v_dot2_f32_f16 / bf16 widening) reduced
//     across the D/8 lanes of a group with DPP; each group keeps its own online
//     softmax state (max, sum, D/8-lane slice of the output) and the groups are
//     merged once at the end of the split.
//   * Page ids are checked on the device before any load through them: an
//     id outside [0, num_pages) stops the split and poisons its log-sum-exp
//     with NaN, so that sequence's output becomes NaN instead of a read out
//     of bounds (two scalar compares per page; nothing measurable).
//   * A split that starts past the sequence end returns before any load
//     (empty windows cost nothing: "[FlyDSL] FP8 MQA logits improvements for
//     gfx950", Changes / Kernel, empty-window fix).  Tokens past the end and
//     page-table entries past the last page are never read.
//
// Each split writes its normalised partial output and its log-sum-exp (base
// 2) to the caller's workspace; the combine kernel merges the splits of a
// sequence as O = sum_s 2^(lse_s - L) o_s with L = log2 sum_s 2^lse_s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mi355_attn {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int PS = kDecodePageSize;

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 dot product of two packed 2-element vectors, accumulated into c
// (v_dot2_f32_f16 / v_dot2_f32_bf16: exact products, fp32 sum).
template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float c) {
  if constexpr (BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                           __builtin_bit_cast(bf16x2_t, y), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), c,
                                  false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf,
                                                            0xf, false));
}

// Sum over each aligned group of G lanes (G = 8 or 16); every lane gets its
// group's total.  quad_perm swaps (xor 1, xor 2), then half-row and row
// mirrors pair each lane with one in the other half of its 8- / 16-lane row.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (G == 16) x += dpp<0x140>(x);  // row_mirror
  return x;
}

// One fp32 -> fp16/bf16 bits, round to nearest even (hardware conversions).
template <bool BF16>
__device__ __forceinline__ uint16_t to_out(float f) {
  if constexpr (BF16) return __builtin_bit_cast(uint16_t, (__bf16)f);
  else return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kDecodeHeadsPerWG) void decode_split_kernel(DecodeArgs a) {
  constexpr int G = D / 8;          // lanes per token row
  constexpr int RPW = 64 / G;       // token rows per wave-wide load
  constexpr int PAGES = 4;          // pages per batch
  constexpr int BATCH = PAGES * PS; // tokens per batch
  constexpr int UNR = BATCH / RPW;  // tokens per lane per batch
  static_assert(UNR * RPW == BATCH, "batch must tile the wave");

  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kDecodeHeadsPerWG + (threadIdx.x >> 6);
  const int split = blockIdx.y;
  const int b = blockIdx.z;
  if (h >= a.H) return;

  // Clamp to the page table's capacity so a bad length cannot index past it.
  const int n = min(a.seq_lens[b], a.max_pages * PS);
  const int t_begin = split * a.tokens_per_split;
  if (t_begin >= n) return;  // empty split: no loads, no writes
  const int t_end = min(n, t_begin + a.tokens_per_split);

  const int grp = lane / G;   // token row within a wave-wide load
  const int gl = lane % G;    // 8-element slice of D
  const int64_t row_stride = (int64_t)a.H * D;            // elements per token
  const int64_t head_off = (int64_t)h * D + gl * 8;

  const u32x4 qv = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.H + h) * D + gl * 8);
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;

  float m = kNegInf, l = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  bool bad_page = false;  // wave-uniform

  for (int tb = t_begin; tb < t_end; tb += BATCH) {
    // Page ids of the pages of this batch; only pages holding a live token
    // are looked up.
    int pgs[PAGES];
    pgs[0] = ptab[tb / PS];
#pragma unroll
    for (int j = 1; j < PAGES; ++j) pgs[j] = (tb + j * PS < t_end) ? ptab[tb / PS + j] : pgs[0];
#pragma unroll
    for (int j = 0; j < PAGES; ++j) bad_page |= (uint32_t)pgs[j] >= (uint32_t)a.num_pages;
    if (bad_page) break;  // no load through an id outside the pool

    u32x4 kr[UNR], vr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int off = grp + RPW * u;  // token offset within the batch
      const int t = tb + off;
      const int pg = pgs[off / PS];
      const int64_t idx = ((int64_t)pg * PS + (off % PS)) * row_stride + head_off;
      if (t < t_end) {
        kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.k_cache + idx));
        vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v_cache + idx));
      } else {
        kr[u] = (u32x4){0u, 0u, 0u, 0u};
        vr[u] = (u32x4){0u, 0u, 0u, 0u};
      }
    }

    float s[UNR];
    float bmax = kNegInf;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) d = dot2<BF16>(qv[j], kr[u][j], d);
      d = group_sum<G>(d) * a.c;
      s[u] = (tb + grp + RPW * u < t_end) ? d : kNegInf;
      bmax = fmaxf(bmax, s[u]);
    }

    const float m_new = fmaxf(m, bmax);
    if (m_new != kNegInf) {  // this group has seen a live token
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // m = -inf -> 0
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float p = __builtin_amdgcn_exp2f(s[u] - m_new);
        l += p;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = __builtin_fmaf(p, lo_f32<BF16>(vr[u][j]), acc[2 * j]);
          acc[2 * j + 1] = __builtin_fmaf(p, hi_f32<BF16>(vr[u][j]), acc[2 * j + 1]);
        }
      }
      m = m_new;
    }
  }

  // Merge the RPW token groups of the wave (lanes gl, gl + G, gl + 2G, ...).
#pragma unroll
  for (int off = G; off < 64; off <<= 1) {
    const float m_o = __shfl_xor(m, off);
    const float l_o = __shfl_xor(l, off);
    const float m_new = fmaxf(m, m_o);
    const float fa = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
    const float fb = (m_o == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_o - m_new);
    l = l * fa + l_o * fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float o = __shfl_xor(acc[e], off);
      acc[e] = acc[e] * fa + o * fb;
    }
    m = m_new;
  }

  // The split holds at least one live token, so l > 0 unless a page id was
  // rejected: then the NaN log-sum-exp carries the error through the combine.
  if (bad_page) {
    if (lane < G) {
      const float nan = __builtin_nanf("");
      float* po = a.part_o + (((int64_t)b * a.H + h) * a.n_splits + split) * D + gl * 8;
      *reinterpret_cast<float4*>(po) = make_float4(nan, nan, nan, nan);
      *reinterpret_cast<float4*>(po + 4) = make_float4(nan, nan, nan, nan);
      if (lane == 0) a.part_lse[((int64_t)b * a.H + h) * a.n_splits + split] = nan;
    }
    return;
  }
  if (lane < G) {
    const float inv = 1.f / l;
    float* po = a.part_o + (((int64_t)b * a.H + h) * a.n_splits + split) * D + gl * 8;
    *reinterpret_cast<float4*>(po) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<float4*>(po + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    if (lane == 0)
      a.part_lse[((int64_t)b * a.H + h) * a.n_splits + split] = m + __log2f(l);
  }
}

// Merge a (sequence, head) row's live splits by log-sum-exp.  A NaN partial
// (rejected page id) makes the output NaN.  OF32: O in fp32.
//
// Eight rows per 64-lane workgroup, eight lanes per row, each lane D/8
// consecutive outputs: a partial row is read as 16-byte loads, the eight
// lanes of a row covering it contiguously, and up to U partials per lane are
// in flight at once (the merge is bound by load latency, not bytes).  Lanes
// first take the row's maximum log-sum-exp over its splits (each lane a
// stride-8 share, reduced over the row's lanes), then accumulate the splits
// in order with the same operations as a one-lane-per-output loop, so the
// result does not depend on this layout.
template <int D, bool BF16, bool OF32>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int E = D / 8;   // outputs per lane
  constexpr int NV = E / 4;  // 16-byte loads per lane per partial (fp32)
  constexpr int U = 8;       // partials loaded per batch
  const int lane = threadIdx.x;
  const int k = lane & 7;                       // the lane's chunk of its row
  const int bh = blockIdx.x * 8 + (lane >> 3);  // the lane's (sequence, head) row
  if (bh >= a.B * a.H) return;                  // whole 8-lane groups leave together
  const int b = bh / a.H;
  const int n = max(0, min(a.seq_lens[b], a.max_pages * PS));
  const int ns = min(a.n_splits, (n + a.tokens_per_split - 1) / a.tokens_per_split);
  const float* lse = a.part_lse + (int64_t)bh * a.n_splits;
  const float* po = a.part_o + (int64_t)bh * a.n_splits * D + k * E;

  float mx = kNegInf;
  int poisoned = 0;
  for (int s = k; s < ns; s += 8) {
    const float l = lse[s];
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
  for (int s0 = 0; s0 < ns; s0 += U) {
    // Loads of the batch (indices past the last split repeat it and are not
    // accumulated).
    float l[U];
    float4 p[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + u, ns - 1);
      l[u] = lse[sp];
#pragma unroll
      for (int v = 0; v < NV; ++v) p[u][v] = *reinterpret_cast<const float4*>(po + sp * D + 4 * v);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < ns) {
        const float w = __builtin_amdgcn_exp2f(l[u] - mx);
        wsum += w;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc[4 * v] = __builtin_fmaf(w, p[u][v].x, acc[4 * v]);
          acc[4 * v + 1] = __builtin_fmaf(w, p[u][v].y, acc[4 * v + 1]);
          acc[4 * v + 2] = __builtin_fmaf(w, p[u][v].z, acc[4 * v + 2]);
          acc[4 * v + 3] = __builtin_fmaf(w, p[u][v].w, acc[4 * v + 3]);
        }
      }
    }
  }
  const float inv = poisoned ? __builtin_nanf("") : (wsum > 0.f ? 1.f / wsum : 0.f);
  const int64_t o0 = (int64_t)bh * D + k * E;
  if constexpr (OF32) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
      *reinterpret_cast<float4*>(static_cast<float*>(a.o) + o0 + 4 * v) =
          make_float4(acc[4 * v] * inv, acc[4 * v + 1] * inv, acc[4 * v + 2] * inv,
                      acc[4 * v + 3] * inv);
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
hipError_t launch_combine_t(bool out_f32, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((a.B * a.H + 7) / 8);
  if (out_f32)
    hipLaunchKernelGGL((decode_combine_kernel<D, BF16, true>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((decode_combine_kernel<D, BF16, false>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_t(bool out_f32, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((a.H + kDecodeHeadsPerWG - 1) / kDecodeHeadsPerWG, a.n_splits, a.B);
  hipLaunchKernelGGL((decode_split_kernel<D, BF16>), grid, dim3(64 * kDecodeHeadsPerWG), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine_t<D, BF16>(out_f32, a, s);
}

}  // namespace

hipError_t launch_decode_combine(int D, bool bf16, bool out_f32, const DecodeArgs& a,
                                 hipStream_t s) {
  if (D == 128) return bf16 ? launch_combine_t<128, true>(out_f32, a, s)
                            : launch_combine_t<128, false>(out_f32, a, s);
  if (D == 64) return bf16 ? launch_combine_t<64, true>(out_f32, a, s)
                           : launch_combine_t<64, false>(out_f32, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_paged_decode(int D, bool bf16, bool out_f32, const DecodeArgs& a,
                               hipStream_t s) {
  if (D == 128) return bf16 ? launch_t<128, true>(out_f32, a, s) : launch_t<128, false>(out_f32, a, s);
  if (D == 64) return bf16 ? launch_t<64, true>(out_f32, a, s) : launch_t<64, false>(out_f32, a, s);
  return hipErrorInvalidValue;
}

}  // namespace mi355_attn
