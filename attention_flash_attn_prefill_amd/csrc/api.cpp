// C ABI of the attention library (include/attn.h): argument validation, launch
// planning and kernel dispatch.  Every check runs before the first HIP call,
// and nothing here allocates, synchronises or reads device memory, so the
// entry points are safe under HIP graph capture (the pages' lesson on launch
// paths that break stream capture: "[FlyDSL] FP8 MQA logits improvements for
// gfx950", Known limitation).
#include "attn.h"

#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace {

using namespace mi355_attn;

constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// dtype = element type of the inputs, optionally OR-ed with ATTN_OUT_F32.
bool parse_dtype(int dtype, bool* bf16, bool* out_f32) {
  const int elt = dtype & ~ATTN_OUT_F32;
  if (elt != ATTN_F16 && elt != ATTN_BF16) return false;
  *bf16 = elt == ATTN_BF16;
  *out_f32 = (dtype & ATTN_OUT_F32) != 0;
  return true;
}

// Softmax scale -> exponent multiplier c = scale * log2(e).  A zero scale
// (uniform weights) becomes the smallest positive normal float, which gives
// the same result (every score * c rounds exp2 to exactly 1) while keeping
// masked scores at -inf rather than -inf * 0 = NaN.
float exp2_multiplier(float scale) {
  const float c = scale * kLog2e;
  return c > 0.f ? c : 1.17549435e-38f;
}

// Paged decode plan (decode_gqa.hip), for every group size g = H / H_kv:
// lines = B x H_kv x ceil(g / 32), each holding its sequence's 32-token tiles;
// the tiles of all lines are cut into W equal ranges on the device, W =
// min(ranges, ceil(NT / min_tiles)) for the batch's actual tile count NT.  A
// range writes one partial row per query of the chunk for every line it
// touches, which the combine reads back, so it covers at least min(g, 32) / 2
// tiles, at most 8 and at least 4: shorter ranges made batches of 1-8
// sequences up to 20% slower (each range also pays a start: the range
// search, then its first tile's latency), longer ones keep fewer loads in
// flight.  Groups of 16 or more query heads take at most half the ranges (4
// resident waves per CU instead of 8): their partials are 16-32 rows per
// range, and halving the ranges ran 7-9% faster at group sizes 16 and 32 on
// batches of 64-256 sequences of up to 8k tokens, no faster at 4 and 8.
// Slots = ranges + lines bound the (range, line) pairs.  The plan depends only
// on host-side sizes; the ranges follow the actual lengths on the device.
struct GqaPlan {
  int ranges, min_tiles, rows_per_slot;
  int64_t lines, slots;
};
GqaPlan plan_gqa(int B, int H, int H_kv, int max_pages, int page_size) {
  GqaPlan p{0, 0, 0, 0, 0};
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || max_pages <= 0 ||
      page_size != kDecodePageSize)
    return p;
  const int group = H / H_kv;
  p.rows_per_slot = group < 32 ? group : 32;
  p.min_tiles = p.rows_per_slot / 2 < 4 ? 4 : (p.rows_per_slot / 2 > 8 ? 8 : p.rows_per_slot / 2);
  p.lines = (int64_t)B * H_kv * ((group + 31) / 32);
  const int64_t max_tiles = ((int64_t)max_pages * page_size + 31) / 32;
  const int64_t nt_max = p.lines * max_tiles;
  if (nt_max >= ((int64_t)1 << 31) || (int64_t)B * H >= ((int64_t)1 << 31) ||
      (int64_t)max_pages * page_size >= ((int64_t)1 << 31))
    return GqaPlan{};
  const int64_t by_size = (nt_max + p.min_tiles - 1) / p.min_tiles;
  const int64_t cap = p.rows_per_slot >= 16 ? kDecodeRanges / 2 : kDecodeRanges;
  p.ranges = (int)(by_size < cap ? by_size : cap);
  p.slots = p.ranges + p.lines;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace mi355_attn {

// Every check of attn_paged_decode_gqa short of the workspace, before any HIP
// call.  ATTN_OK with *need = 0: nothing to launch (B * H = 0).  ATTN_OK with
// *need > 0: a launch needs that many workspace bytes.
int check_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, const int32_t* seq_lens, const void* o, int B,
                       int H, int H_kv, int D, int page_size, int num_pages,
                       int max_pages_per_seq, int dtype, float scale, size_t* need) {
  *need = 0;
  if (B < 0 || H < 0 || H_kv < 0 || num_pages < 0 || max_pages_per_seq < 0) return ATTN_E_INVALID;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return ATTN_E_INVALID;
  bool bf16, out_f32;
  if (!parse_dtype(dtype, &bf16, &out_f32)) return ATTN_E_INVALID;
  if (!isfinite(scale) || scale < 0.f) return ATTN_E_INVALID;
  if (D != 64 && D != 128) return D <= 0 ? ATTN_E_INVALID : ATTN_E_UNSUPPORTED;
  if (page_size != kDecodePageSize) return page_size <= 0 ? ATTN_E_INVALID : ATTN_E_UNSUPPORTED;
  if ((int64_t)B * H == 0) return ATTN_OK;
  if ((int64_t)max_pages_per_seq * page_size >= ((int64_t)1 << 31))
    return ATTN_E_UNSUPPORTED;  // token positions are 32-bit
  if (num_pages == 0 || max_pages_per_seq == 0) return ATTN_E_INVALID;  // seq_len >= 1 needs a page
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !o) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return ATTN_E_INVALID;
  if (((uintptr_t)page_table & 3u) || ((uintptr_t)seq_lens & 3u)) return ATTN_E_INVALID;

  if (plan_gqa(B, H, H_kv, max_pages_per_seq, page_size).ranges == 0)
    return ATTN_E_UNSUPPORTED;  // index limits
  *need = attn_paged_decode_gqa_workspace_size(B, H, H_kv, D, max_pages_per_seq, page_size);
  return *need > 0 ? ATTN_OK : ATTN_E_UNSUPPORTED;
}

}  // namespace mi355_attn

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_INVALID: return "invalid argument";
    case ATTN_E_UNSUPPORTED: return "unsupported configuration";
    case ATTN_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int attn_prefill(const void* q, const void* k, const void* v, void* o, int B, int H, int Sq,
                 int Skv, int D, int layout, int dtype, int causal, float scale,
                 hipStream_t stream) {
  return attn_prefill_gqa(q, k, v, o, B, H, H, Sq, Skv, D, layout, dtype, causal, scale, stream);
}

int attn_prefill_gqa(const void* q, const void* k, const void* v, void* o, int B, int H,
                     int H_kv, int Sq, int Skv, int D, int layout, int dtype, int causal,
                     float scale, hipStream_t stream) {
  return attn_prefill_lse(q, k, v, o, nullptr, B, H, H_kv, Sq, Skv, D, layout, dtype, causal,
                          scale, stream);
}

}  // extern "C"

namespace {

// Every check of a dense prefill and its kernel arguments, before any HIP
// call.  ATTN_OK with *run = false: nothing to compute.
int prepare_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int H_kv, int Sq, int Skv, int D, int layout, int dtype,
                    float scale, PrefillArgs* ap, bool* bf16_out, bool* out_f32_out,
                    bool* run) {
  *run = false;
  if (B < 0 || H < 0 || H_kv < 0 || Sq < 0 || Skv < 0) return ATTN_E_INVALID;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return ATTN_E_INVALID;
  if (layout != ATTN_BHSD && layout != ATTN_BSHD) return ATTN_E_INVALID;
  bool bf16, out_f32;
  if (!parse_dtype(dtype, &bf16, &out_f32)) return ATTN_E_INVALID;
  if (!isfinite(scale) || scale < 0.f) return ATTN_E_INVALID;
  if (D != 64 && D != 128) return D <= 0 ? ATTN_E_INVALID : ATTN_E_UNSUPPORTED;
  if ((int64_t)B * H * Sq == 0) return ATTN_OK;  // nothing to compute
  if (!q || !o) return ATTN_E_INVALID;
  if (Skv > 0 && (!k || !v)) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(o) || (Skv > 0 && (!aligned16(k) || !aligned16(v))))
    return ATTN_E_INVALID;
  if ((uintptr_t)lse & 3u) return ATTN_E_INVALID;

  // In-head offsets (row * row_stride) are 32-bit in the kernel.
  const int64_t q_row = layout == ATTN_BHSD ? D : (int64_t)H * D;
  const int64_t kv_row = layout == ATTN_BHSD ? D : (int64_t)H_kv * D;
  if ((int64_t)Sq * q_row >= ((int64_t)1 << 31) || (int64_t)Skv * kv_row >= ((int64_t)1 << 31))
    return ATTN_E_UNSUPPORTED;
  // Byte offsets inside a 64-row tile are 32-bit too.
  if (q_row >= ((int64_t)1 << 24) || kv_row >= ((int64_t)1 << 24)) return ATTN_E_UNSUPPORTED;
  if ((int64_t)B * H * ((Sq + 127) / 128) >= ((int64_t)1 << 31)) return ATTN_E_UNSUPPORTED;

  PrefillArgs& a = *ap;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.H = H;
  a.H_kv = H_kv;
  a.group = H / H_kv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.n_mtiles = 0;     // set by launch_prefill for the chosen tile shape
  a.total_tiles = 0;
  if (layout == ATTN_BHSD) {
    a.q_sb = (int64_t)H * Sq * D; a.q_sh = (int64_t)Sq * D; a.q_ss = D;
    a.k_sb = (int64_t)H_kv * Skv * D; a.k_sh = (int64_t)Skv * D; a.k_ss = D;
  } else {
    a.q_sb = (int64_t)Sq * H * D; a.q_sh = D; a.q_ss = H * D;
    a.k_sb = (int64_t)Skv * H_kv * D; a.k_sh = D; a.k_ss = H_kv * D;
  }
  a.c = exp2_multiplier(scale);
  a.o_scale = 1.f;
  a.causal_off = Skv - Sq;
  a.k_cache = a.v_cache = nullptr;
  a.page_table = a.prefix_lens = a.qo_start = nullptr;
  a.max_pages = a.num_pages = a.total_tokens = 0;
  a.lse = lse;
  a.n_splits = 1;
  a.split_tiles = (Skv + 63) / 64;
  a.split_o_stride = a.split_lse_stride = 0;
  *bf16_out = bf16;
  *out_f32_out = out_f32;
  *run = true;
  return ATTN_OK;
}

// Split-KV plans of attn_prefill_splitkv and attn_extend_splitkv, from sizes
// only.  Work items are the plain grid's workgroups (prefill: batch, head,
// query tile of 256 rows, 128 for D = 64; extend: below); each item's keys
// are cut into n ranges of `split_tiles` 64-key tiles, at least 8 tiles
// (512 keys) each.  A split is considered only when the plain grid holds fewer
// than two workgroups per CU (above that the plain causal grid pairs its
// tiles) and there are at least 16 key tiles.  The plan takes the n with the
// least modelled time, the smallest n on a tie.  The model, fitted to
// measured split and plain prefill times:
//   * the split kernel takes as long as its busiest CU, which holds w =
//     ceil(items * n / 256) workgroups (run one after another at D = 128,
//     where one workgroup of 8 waves fills a CU; up to three at a time at
//     D = 64, 4 waves each); each costs its key tiles at the per-CU tile time
//     (D = 128: 2.1 us; D = 64: 0.8 us with three workgroups resident, 4.5%
//     more with two, 22% more with one) plus, at D = 64, ~3 us of its own
//     (Q loads, the epilogue);
//   * for n > 1, every split's fp32 partials (O and LSE of each query row,
//     written by the split kernel and read back by the combine) at 5.5 TB/s,
//     plus the combine's launch (~5 us).
struct SplitKvPlan {
  int n_splits, split_tiles;
};
// The model over items work items of n_kt key tiles each, rows_total query
// rows (times heads) of partials per split.
SplitKvPlan plan_splits_modelled(int64_t items, int64_t n_kt, double rows_total, int D) {
  constexpr int64_t kMinSplitTiles = 8;
  const SplitKvPlan none{1, (int)n_kt};
  if (items <= 0 || items >= 2 * kNumCUs || n_kt < 2 * kMinSplitTiles) return none;
  const double split_us = rows_total * (D + 1) * 8 / 5.5e6;
  constexpr double kCombineUs = 5.0;
  auto cost = [&](int64_t n, int64_t tiles) {
    const int64_t w = (items * n + kNumCUs - 1) / kNumCUs;
    double per_wg;
    if (D == 128) {
      per_wg = 2.1 * (double)tiles;
    } else {
      const double occ = w >= 3 ? 1.0 : (w == 2 ? 1.045 : 1.22);
      per_wg = 0.8 * occ * (double)tiles + 3.0;
    }
    const double t = (double)w * per_wg;
    return n > 1 ? t + (double)n * split_us + kCombineUs : t;
  };
  SplitKvPlan best = none;
  double best_t = cost(1, n_kt);
  const int64_t n_cap = 16 * kNumCUs;
  const int64_t n_max = n_kt / kMinSplitTiles < n_cap ? n_kt / kMinSplitTiles : n_cap;
  for (int64_t n = 2; n <= n_max; ++n) {
    const int64_t tiles = (n_kt + n - 1) / n;
    const int64_t ns = (n_kt + tiles - 1) / tiles;  // ranges actually used
    const double t = cost(ns, tiles);
    if (t < best_t) {
      best_t = t;
      best = SplitKvPlan{(int)ns, (int)tiles};
    }
  }
  return best;
}

SplitKvPlan plan_prefill_splitkv(int B, int H, int Sq, int Skv, int D) {
  const int64_t rows = D == 128 ? 256 : 128;
  const int64_t items = (int64_t)B * H * ((Sq + rows - 1) / rows);
  return plan_splits_modelled(items, ((int64_t)Skv + 63) / 64, (double)B * H * Sq, D);
}

// Split-KV extend: units (sequence, KV head, head group, query tile) as in
// attn_extend's grid, sized from the bounds max_extend_len and the prefix
// capacity max_pages_per_seq * 16 (a unit walks its prefix tiles, then its
// new tokens' tiles); the partials cover total_tokens rows of every head.
SplitKvPlan plan_extend_splitkv(int B, int H, int H_kv, int D, int total_tokens,
                                int max_extend_len, int max_pages_per_seq) {
  const int hpw = (H / H_kv) % 4 == 0 ? 4 : 1;
  const int64_t rpw = (D == 128 ? 256 : 128) / hpw;
  const int64_t items = (int64_t)B * (H / hpw) * ((max_extend_len + rpw - 1) / rpw);
  const int64_t n_kt = ((int64_t)max_pages_per_seq * kDecodePageSize + 63) / 64 +
                       ((int64_t)max_extend_len + 63) / 64;
  return plan_splits_modelled(items, n_kt, (double)total_tokens * H, D);
}

}  // namespace

// Argument checks and kernel arguments of attn_extend (shared with
// attn_extend_splitkv).  *run is false when there is nothing to compute.
static int prepare_extend(const void* q, const void* k, const void* v, const void* k_cache,
                          const void* v_cache, const int32_t* page_table,
                          const int32_t* prefix_lens, const int32_t* qo_start, void* o, int B,
                          int H, int H_kv, int D, int total_tokens, int max_extend_len,
                          int page_size, int num_pages, int max_pages_per_seq, int dtype,
                          float scale, PrefillArgs* out, bool* bf16_out, bool* out_f32_out,
                          bool* run) {
  *run = false;
  if (B < 0 || H < 0 || H_kv < 0 || total_tokens < 0 || max_extend_len < 0 || num_pages < 0 ||
      max_pages_per_seq < 0)
    return ATTN_E_INVALID;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return ATTN_E_INVALID;
  bool bf16, out_f32;
  if (!parse_dtype(dtype, &bf16, &out_f32)) return ATTN_E_INVALID;
  if (!isfinite(scale) || scale < 0.f) return ATTN_E_INVALID;
  if (D != 64 && D != 128) return D <= 0 ? ATTN_E_INVALID : ATTN_E_UNSUPPORTED;
  if (page_size != kDecodePageSize) return page_size <= 0 ? ATTN_E_INVALID : ATTN_E_UNSUPPORTED;
  if ((int64_t)B * H * max_extend_len == 0 || total_tokens == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !qo_start) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_E_INVALID;
  if ((uintptr_t)qo_start & 3u) return ATTN_E_INVALID;
  if (max_pages_per_seq > 0) {  // prefixes may exist: the cache must be there
    if (num_pages == 0 || !k_cache || !v_cache || !page_table || !prefix_lens)
      return ATTN_E_INVALID;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return ATTN_E_INVALID;
    if (((uintptr_t)page_table & 3u) || ((uintptr_t)prefix_lens & 3u)) return ATTN_E_INVALID;
  }
  // Row offsets within a sequence's new tokens are 32-bit in the kernel, and
  // so are key positions (prefix plus new tokens).
  if ((int64_t)max_extend_len * H * D * 2 >= ((int64_t)1 << 31)) return ATTN_E_UNSUPPORTED;
  if ((int64_t)max_pages_per_seq * kDecodePageSize + max_extend_len >= ((int64_t)1 << 31))
    return ATTN_E_UNSUPPORTED;
  if ((int64_t)kDecodePageSize * H_kv * D * 2 >= ((int64_t)1 << 31)) return ATTN_E_UNSUPPORTED;

  PrefillArgs& a = *out;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.H = H;
  a.H_kv = H_kv;
  a.group = H / H_kv;
  a.Sq = max_extend_len;  // bounds every sequence's new tokens; sets the grid
  a.Skv = 0;
  a.causal_off = 0;
  a.n_mtiles = 0;
  a.total_tiles = 0;
  a.q_sb = 0; a.q_sh = D; a.q_ss = H * D;          // [T, H, D]
  a.k_sb = 0; a.k_sh = D; a.k_ss = H_kv * D;       // [T, H_kv, D]
  a.c = exp2_multiplier(scale);
  a.o_scale = 1.f;
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.page_table = page_table;
  a.prefix_lens = prefix_lens;
  a.qo_start = qo_start;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.total_tokens = total_tokens;
  a.lse = nullptr;
  a.n_splits = 1;
  a.split_tiles = 0;
  a.split_o_stride = a.split_lse_stride = 0;
  *bf16_out = bf16;
  *out_f32_out = out_f32;
  *run = true;
  return ATTN_OK;
}

extern "C" {

int attn_prefill_lse(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int H_kv, int Sq, int Skv, int D, int layout, int dtype, int causal,
                     float scale, hipStream_t stream) {
  PrefillArgs a;
  bool bf16 = false, out_f32 = false, run = false;
  const int st = prepare_prefill(q, k, v, o, lse, B, H, H_kv, Sq, Skv, D, layout, dtype, scale, &a,
                                 &bf16, &out_f32, &run);
  if (st != ATTN_OK || !run) return st;
  hipError_t e = launch_prefill(D, bf16, causal != 0, out_f32, a, B, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

size_t attn_prefill_splitkv_workspace_size(int B, int H, int Sq, int Skv, int D) {
  if (B < 0 || H < 0 || Sq < 0 || Skv < 0 || (D != 64 && D != 128)) return 0;
  const SplitKvPlan p = plan_prefill_splitkv(B, H, Sq, Skv, D);
  if (p.n_splits <= 1) return 0;
  const size_t rows = (size_t)B * H * Sq;
  return (size_t)p.n_splits * (align256(rows * D * sizeof(float)) + align256(rows * sizeof(float)));
}

int attn_prefill_splitkv_num_splits(int B, int H, int Sq, int Skv, int D) {
  if (B < 0 || H < 0 || Sq < 0 || Skv < 0 || (D != 64 && D != 128)) return 0;
  return plan_prefill_splitkv(B, H, Sq, Skv, D).n_splits;
}

int attn_prefill_splitkv(const void* q, const void* k, const void* v, void* o, int B, int H,
                         int H_kv, int Sq, int Skv, int D, int layout, int dtype, int causal,
                         float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  PrefillArgs a;
  bool bf16 = false, out_f32 = false, run = false;
  const int st = prepare_prefill(q, k, v, o, nullptr, B, H, H_kv, Sq, Skv, D, layout, dtype,
                                 scale, &a, &bf16, &out_f32, &run);
  if (st != ATTN_OK || !run) return st;
  const SplitKvPlan p = plan_prefill_splitkv(B, H, Sq, Skv, D);
  if (p.n_splits <= 1) {  // the grid fills the GPU: the plain prefill
    hipError_t e = launch_prefill(D, bf16, causal != 0, out_f32, a, B, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  }
  const size_t need = attn_prefill_splitkv_workspace_size(B, H, Sq, Skv, D);
  if (!workspace || workspace_bytes < need) return ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_E_INVALID;
  const size_t rows = (size_t)B * H * Sq;
  a.n_splits = p.n_splits;
  a.split_tiles = p.split_tiles;
  a.split_o_stride = (int64_t)rows * D;
  a.split_lse_stride = (int64_t)rows;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             p.n_splits * align256(rows * D * sizeof(float)));
  hipError_t e = launch_prefill_splitkv(D, bf16, causal != 0, out_f32, a, B, part_o, part_lse,
                                        stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

// Two fp32 arrays of B*H*Sq (delta, then -LSE log2 e), each padded to 256 bytes.
static size_t bwd_row_array_bytes(int B, int H, int Sq) {
  return (((size_t)B * H * Sq * sizeof(float)) + 255) & ~(size_t)255;
}

size_t attn_prefill_bwd_workspace_size(int B, int H, int Sq) {
  if (B < 0 || H < 0 || Sq < 0) return 0;
  return 2 * bwd_row_array_bytes(B, H, Sq);
}

int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv,
                     int Sq, int Skv, int D, int layout, int dtype, int causal, float scale,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || H < 0 || H_kv < 0 || Sq < 0 || Skv < 0) return ATTN_E_INVALID;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return ATTN_E_INVALID;
  if (layout != ATTN_BHSD && layout != ATTN_BSHD) return ATTN_E_INVALID;
  bool bf16, out_f32;
  if (!parse_dtype(dtype, &bf16, &out_f32)) return ATTN_E_INVALID;
  if (!isfinite(scale) || scale < 0.f) return ATTN_E_INVALID;
  if (D != 64 && D != 128) return D <= 0 ? ATTN_E_INVALID : ATTN_E_UNSUPPORTED;
  if ((int64_t)B * H == 0 || ((int64_t)Sq == 0 && (int64_t)Skv == 0)) return ATTN_OK;
  if (Sq > 0 && (!q || !o || !dO || !lse || !dq)) return ATTN_E_INVALID;
  if (Skv > 0 && (!k || !v || !dk || !dv)) return ATTN_E_INVALID;
  for (const void* p : {q, k, v, o, dO, (const void*)dq, (const void*)dk, (const void*)dv})
    if (p && !aligned16(p)) return ATTN_E_INVALID;
  if ((uintptr_t)lse & 3u) return ATTN_E_INVALID;
  const size_t need = attn_prefill_bwd_workspace_size(B, H, Sq);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;
  if (workspace && !aligned16(workspace)) return ATTN_E_INVALID;
  const int64_t q_row = layout == ATTN_BHSD ? D : (int64_t)H * D;
  const int64_t kv_row = layout == ATTN_BHSD ? D : (int64_t)H_kv * D;
  if ((int64_t)Sq * q_row >= ((int64_t)1 << 31) || (int64_t)Skv * kv_row >= ((int64_t)1 << 31))
    return ATTN_E_UNSUPPORTED;
  if (q_row >= ((int64_t)1 << 24) || kv_row >= ((int64_t)1 << 24)) return ATTN_E_UNSUPPORTED;
  // Grids: delta (16 rows per workgroup), dK/dV (128 keys), dQ (128 or 256 queries).
  const int64_t grid_limit = (int64_t)1 << 31;
  if ((int64_t)B * H * Sq / 16 >= grid_limit ||
      (int64_t)B * H_kv * ((Skv + 127) / 128) >= grid_limit ||
      (int64_t)B * H * ((Sq + 127) / 128) >= grid_limit)
    return ATTN_E_UNSUPPORTED;

  BackwardArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dO = static_cast<const uint16_t*>(dO);
  a.lse = lse;
  a.delta = static_cast<float*>(workspace);
  a.nl2 = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                   bwd_row_array_bytes(B, H, Sq));
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.group = H / H_kv;
  a.Sq = Sq;
  a.Skv = Skv;
  if (layout == ATTN_BHSD) {
    a.q_sb = (int64_t)H * Sq * D; a.q_sh = (int64_t)Sq * D; a.q_ss = D;
    a.k_sb = (int64_t)H_kv * Skv * D; a.k_sh = (int64_t)Skv * D; a.k_ss = D;
  } else {
    a.q_sb = (int64_t)Sq * H * D; a.q_sh = D; a.q_ss = H * D;
    a.k_sb = (int64_t)Skv * H_kv * D; a.k_sh = D; a.k_ss = H_kv * D;
  }
  a.scale = scale;
  a.c = exp2_multiplier(scale);  // the forward's multiplier: P matches its LSE
  a.causal_off = Skv - Sq;
  a.n_tiles = a.total = 0;
  hipError_t e = launch_prefill_backward(D, bf16, causal != 0, out_f32, a, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_prefill_fp8(const void* q, const void* k, const void* v, void* o, int B, int H,
                     int H_kv, int Sq, int Skv, int D, int layout, int out_dtype, int causal,
                     float scale, float q_descale, float k_descale, float v_descale,
                     hipStream_t stream) {
  if (B < 0 || H < 0 || H_kv < 0 || Sq < 0 || Skv < 0) return ATTN_E_INVALID;
  if (H > 0 && (H_kv == 0 || H % H_kv != 0)) return ATTN_E_INVALID;
  if (layout != ATTN_BHSD && layout != ATTN_BSHD) return ATTN_E_INVALID;
  bool out_bf16, out_f32;
  if (!parse_dtype(out_dtype, &out_bf16, &out_f32)) return ATTN_E_INVALID;
  if (!isfinite(scale) || scale < 0.f) return ATTN_E_INVALID;
  for (float d : {q_descale, k_descale, v_descale})
    if (!isfinite(d) || d < 0.f) return ATTN_E_INVALID;
  if (D != 64 && D != 128) return D <= 0 ? ATTN_E_INVALID : ATTN_E_UNSUPPORTED;
  if ((int64_t)B * H * Sq == 0) return ATTN_OK;
  if (!q || !o) return ATTN_E_INVALID;
  if (Skv > 0 && (!k || !v)) return ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(o) || (Skv > 0 && (!aligned16(k) || !aligned16(v))))
    return ATTN_E_INVALID;
  const int64_t q_row = layout == ATTN_BHSD ? D : (int64_t)H * D;
  const int64_t kv_row = layout == ATTN_BHSD ? D : (int64_t)H_kv * D;
  if ((int64_t)Sq * q_row * 4 >= ((int64_t)1 << 31) || (int64_t)Skv * kv_row >= ((int64_t)1 << 31))
    return ATTN_E_UNSUPPORTED;
  if (q_row >= ((int64_t)1 << 24) || kv_row >= ((int64_t)1 << 24)) return ATTN_E_UNSUPPORTED;
  if ((int64_t)B * H * ((Sq + 127) / 128) >= ((int64_t)1 << 31)) return ATTN_E_UNSUPPORTED;

  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);  // e4m3fn bytes; the kernel addresses them bytewise
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.H = H;
  a.H_kv = H_kv;
  a.group = H / H_kv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.n_mtiles = 0;
  a.total_tiles = 0;
  if (layout == ATTN_BHSD) {
    a.q_sb = (int64_t)H * Sq * D; a.q_sh = (int64_t)Sq * D; a.q_ss = D;
    a.k_sb = (int64_t)H_kv * Skv * D; a.k_sh = (int64_t)Skv * D; a.k_ss = D;
  } else {
    a.q_sb = (int64_t)Sq * H * D; a.q_sh = D; a.q_ss = H * D;
    a.k_sb = (int64_t)Skv * H_kv * D; a.k_sh = D; a.k_ss = H_kv * D;
  }
  // The q and k descales multiply every score: fold them into the exponent
  // multiplier; the v descale multiplies O.
  a.c = exp2_multiplier(scale * q_descale * k_descale);
  a.o_scale = v_descale;
  a.causal_off = Skv - Sq;
  a.k_cache = a.v_cache = nullptr;
  a.page_table = a.prefix_lens = a.qo_start = nullptr;
  a.max_pages = a.num_pages = a.total_tokens = 0;
  a.lse = nullptr;
  hipError_t e = launch_prefill_fp8(D, out_bf16, causal != 0, out_f32, a, B, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_extend(const void* q, const void* k, const void* v, const void* k_cache,
                const void* v_cache, const int32_t* page_table, const int32_t* prefix_lens,
                const int32_t* qo_start, void* o, int B, int H, int H_kv, int D,
                int total_tokens, int max_extend_len, int page_size, int num_pages,
                int max_pages_per_seq, int dtype, float scale, hipStream_t stream) {
  PrefillArgs a;
  bool bf16 = false, out_f32 = false, run = false;
  const int st = prepare_extend(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, o,
                                B, H, H_kv, D, total_tokens, max_extend_len, page_size,
                                num_pages, max_pages_per_seq, dtype, scale, &a, &bf16, &out_f32,
                                &run);
  if (st != ATTN_OK || !run) return st;
  hipError_t e = launch_extend(D, bf16, out_f32, a, B, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

static bool extend_sizes_ok(int B, int H, int H_kv, int D, int total_tokens, int max_extend_len,
                            int max_pages_per_seq) {
  return B >= 0 && H >= 0 && H_kv >= 0 && total_tokens >= 0 && max_extend_len >= 0 &&
         max_pages_per_seq >= 0 && (H == 0 || (H_kv > 0 && H % H_kv == 0)) &&
         (D == 64 || D == 128);
}

int attn_extend_splitkv_num_splits(int B, int H, int H_kv, int D, int total_tokens,
                                   int max_extend_len, int max_pages_per_seq) {
  if (!extend_sizes_ok(B, H, H_kv, D, total_tokens, max_extend_len, max_pages_per_seq)) return 0;
  if ((int64_t)B * H * max_extend_len == 0 || total_tokens == 0) return 1;
  return plan_extend_splitkv(B, H, H_kv, D, total_tokens, max_extend_len, max_pages_per_seq)
      .n_splits;
}

size_t attn_extend_splitkv_workspace_size(int B, int H, int H_kv, int D, int total_tokens,
                                          int max_extend_len, int max_pages_per_seq) {
  const int n = attn_extend_splitkv_num_splits(B, H, H_kv, D, total_tokens, max_extend_len,
                                               max_pages_per_seq);
  if (n <= 1) return 0;
  const size_t rows = (size_t)total_tokens * H;
  return (size_t)n * (align256(rows * D * sizeof(float)) + align256(rows * sizeof(float)));
}

int attn_extend_splitkv(const void* q, const void* k, const void* v, const void* k_cache,
                        const void* v_cache, const int32_t* page_table,
                        const int32_t* prefix_lens, const int32_t* qo_start, void* o, int B,
                        int H, int H_kv, int D, int total_tokens, int max_extend_len,
                        int page_size, int num_pages, int max_pages_per_seq, int dtype,
                        float scale, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  PrefillArgs a;
  bool bf16 = false, out_f32 = false, run = false;
  const int st = prepare_extend(q, k, v, k_cache, v_cache, page_table, prefix_lens, qo_start, o,
                                B, H, H_kv, D, total_tokens, max_extend_len, page_size,
                                num_pages, max_pages_per_seq, dtype, scale, &a, &bf16, &out_f32,
                                &run);
  if (st != ATTN_OK || !run) return st;
  const SplitKvPlan p =
      plan_extend_splitkv(B, H, H_kv, D, total_tokens, max_extend_len, max_pages_per_seq);
  if (p.n_splits <= 1) {  // the grid fills the GPU: the plain extend
    hipError_t e = launch_extend(D, bf16, out_f32, a, B, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  }
  const size_t need = attn_extend_splitkv_workspace_size(B, H, H_kv, D, total_tokens,
                                                         max_extend_len, max_pages_per_seq);
  if (!workspace || workspace_bytes < need) return ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_E_INVALID;
  const size_t rows = (size_t)total_tokens * H;
  a.n_splits = p.n_splits;
  a.split_tiles = p.split_tiles;
  a.split_o_stride = (int64_t)rows * D;
  a.split_lse_stride = (int64_t)rows;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             p.n_splits * align256(rows * D * sizeof(float)));
  hipError_t e = launch_extend_splitkv(D, bf16, out_f32, a, B, part_o, part_lse, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_paged_decode_gqa_num_splits(int B, int H, int H_kv, int max_pages_per_seq,
                                     int page_size, int* tokens_per_split) {
  const GqaPlan g = plan_gqa(B, H, H_kv, max_pages_per_seq, page_size);
  if (tokens_per_split) *tokens_per_split = g.ranges > 0 ? g.min_tiles * 32 : 0;
  return g.ranges;
}

int attn_paged_decode_num_splits(int B, int H, int max_pages_per_seq, int page_size,
                                 int* tokens_per_split) {
  return attn_paged_decode_gqa_num_splits(B, H, H, max_pages_per_seq, page_size,
                                          tokens_per_split);
}

size_t attn_paged_decode_gqa_workspace_size(int B, int H, int H_kv, int D, int max_pages_per_seq,
                                            int page_size) {
  if (D != 64 && D != 128) return 0;
  // partial outputs [slots, rows, D], log-sum-exps [slots, rows], then the
  // range metadata (B + 3 ints), each 256-B aligned
  const GqaPlan g = plan_gqa(B, H, H_kv, max_pages_per_seq, page_size);
  if (g.ranges == 0) return 0;
  const size_t rows = (size_t)g.slots * g.rows_per_slot;
  return align256(rows * D * sizeof(float)) + align256(rows * sizeof(float)) +
         ((size_t)B + 3) * sizeof(int);
}

size_t attn_paged_decode_workspace_size(int B, int H, int D, int max_pages_per_seq,
                                        int page_size) {
  return attn_paged_decode_gqa_workspace_size(B, H, H, D, max_pages_per_seq, page_size);
}

int attn_paged_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* page_table, const int32_t* seq_lens, void* o, int B,
                          int H, int H_kv, int D, int page_size, int num_pages,
                          int max_pages_per_seq, int dtype, float scale, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  const int st = mi355_attn::check_paged_decode(q, k_cache, v_cache, page_table, seq_lens, o, B,
                                                H, H_kv, D, page_size, num_pages,
                                                max_pages_per_seq, dtype, scale, &need);
  if (st != ATTN_OK || need == 0) return st;
  if (!workspace || workspace_bytes < need) return ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_E_INVALID;
  bool bf16, out_f32;
  parse_dtype(dtype, &bf16, &out_f32);
  const int group = H / H_kv;
  const int qchunks = (group + 31) / 32;
  const GqaPlan g = plan_gqa(B, H, H_kv, max_pages_per_seq, page_size);

  const size_t rows = (size_t)g.slots * g.rows_per_slot;
  const size_t o_bytes = align256(rows * D * sizeof(float));
  DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.o = o;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  a.meta = reinterpret_cast<int*>(static_cast<char*>(workspace) + o_bytes +
                                  align256(rows * sizeof(float)));
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.group = group;
  a.qchunks = qchunks;
  a.max_pages = max_pages_per_seq;
  a.n_splits = g.ranges;
  a.min_tiles = g.min_tiles;
  a.rows_per_slot = g.rows_per_slot;
  a.num_pages = num_pages;
  a.c = exp2_multiplier(scale);
  hipError_t e = launch_paged_decode_gqa(D, bf16, out_f32, a, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* page_table, const int32_t* seq_lens, void* o, int B, int H,
                      int D, int page_size, int num_pages, int max_pages_per_seq, int dtype,
                      float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attn_paged_decode_gqa(q, k_cache, v_cache, page_table, seq_lens, o, B, H, H, D,
                               page_size, num_pages, max_pages_per_seq, dtype, scale, workspace,
                               workspace_bytes, stream);
}

}  // extern "C"
