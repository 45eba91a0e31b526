// Internal interface between the C-ABI host code (api.cpp) and the HIP kernel
// translation units (prefill.hip, decode_gqa.hip, backward.hip).  Not installed; not
// part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mi355_attn {

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;             // fp16/bf16 like q, or fp32 (out_f32)
  int H, Sq, Skv;       // H query heads
  int H_kv, group;     // KV heads and query heads per KV head (H = H_kv * group)
  int n_mtiles;        // ceil(Sq / BM), set by launch_prefill
  int pair_tiles;      // causal: one workgroup per pair of query tiles, set by launch_prefill
  int total_tiles;     // grid size (work items), set by launch_prefill
  int64_t q_sb, q_sh;  // element strides of q and o between batches / heads
  int q_ss;            // element stride between query rows
  int64_t k_sb, k_sh;  // element strides of k and v (per batch, per KV head)
  int k_ss;
  float c;             // scale * log2(e) (fp8: times the q and k descales)
  float o_scale;       // factor on O (fp8: the v descale; else 1)
  int causal_off;      // Skv - Sq (bottom-right causal alignment)
  // Extend kernels only: the new tokens of sequence b are rows qo_start[b] ..
  // qo_start[b+1]-1 of q, k, v, o (token-major, Sq = max_extend_len bounds
  // them), and its first prefix_lens[b] keys come from a paged cache
  // [num_pages, 16, H_kv, D] through page_table [B, max_pages].
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* prefix_lens;
  const int32_t* qo_start;
  int max_pages, num_pages, total_tokens;
  // Forward only: if not null, the natural log-sum-exp of each query row's
  // scaled logits, [B, H, Sq] fp32 (-inf for a row with no visible key).
  float* lse;
  // Split-KV prefill and extend only: the keys of each query tile are cut
  // into n_splits ranges of split_tiles 64-key tiles.
  int n_splits, split_tiles;
  int64_t split_o_stride, split_lse_stride;  // elements between the partials' planes
};

hipError_t launch_prefill(int D, bool bf16, bool causal, bool out_f32, const PrefillArgs& a,
                          int B, hipStream_t s);
// Split-KV prefill: the split kernel writes partial O (fp32, q's strides)
// and log-sum-exps per key range into part_o / part_lse (n_splits planes of
// B*H*Sq*D and B*H*Sq floats), then a combine kernel merges them into a.o.
hipError_t launch_prefill_splitkv(int D, bool bf16, bool causal, bool out_f32,
                                  const PrefillArgs& a, int B, float* part_o, float* part_lse,
                                  hipStream_t s);
// FP8 (e4m3fn) q, k, v: Q.K^T on the fp8 MFMA, V widened to fp16 on staging;
// O in fp16 (out_bf16 = false), bf16 or fp32.  Strides are in elements (bytes).
hipError_t launch_prefill_fp8(int D, bool out_bf16, bool causal, bool out_f32,
                              const PrefillArgs& a, int B, hipStream_t s);
// Backward of dense prefill (fp16/bf16, BHSD/BSHD, grouped heads, causal).
struct BackwardArgs {
  const uint16_t* q;    // [B, H, Sq, D] / [B, Sq, H, D]
  const uint16_t* k;    // H_kv heads, Skv keys
  const uint16_t* v;
  const uint16_t* o;    // forward output, like q
  const uint16_t* dO;   // like q
  const float* lse;     // [B, H, Sq] natural log-sum-exp from the forward
  float* delta;         // [B, H, Sq] workspace: rowsum(dO * O)
  float* nl2;           // [B, H, Sq] workspace: -LSE * log2(e) (-inf for a row with no key)
  void* dq;             // like q (dtype, or fp32 with out_f32)
  void* dk;             // like k
  void* dv;             // like v
  int B, H, H_kv, group, Sq, Skv;
  int64_t q_sb, q_sh;   // element strides of q, o, dO, dq
  int q_ss;
  int64_t k_sb, k_sh;   // element strides of k, v, dk, dv
  int k_ss;
  float scale;          // softmax scale
  float c;              // scale * log2(e)
  int causal_off;       // Skv - Sq
  int n_tiles, total;   // set by the launcher
};
hipError_t launch_prefill_backward(int D, bool bf16, bool causal, bool out_f32,
                                   const BackwardArgs& a, hipStream_t s);

// Extend attention (causal over a paged prefix followed by the new tokens).
hipError_t launch_extend(int D, bool bf16, bool out_f32, const PrefillArgs& a, int B,
                         hipStream_t s);
// Split-KV extend: the extend kernel over n_splits ranges of split_tiles key
// tiles of each unit (prefix tiles first, then the new tokens'), partial O
// (fp32, q's strides) and log-sum-exps ([H, total_tokens] per plane) into
// part_o / part_lse, then a combine into a.o of the rows attn_extend writes.
hipError_t launch_extend_splitkv(int D, bool bf16, bool out_f32, const PrefillArgs& a, int B,
                                 float* part_o, float* part_lse, hipStream_t s);

// Paged decode (decode_gqa.hip).  H query heads share H_kv KV heads (group =
// H / H_kv, 1 for multi-head attention): one wave per work range of the
// batch's (sequence, KV head, chunk of up to 32 query heads) lines.
constexpr int kDecodePageSize = 16;
constexpr int kNumCUs = 256;  // compute units of an MI355X (8 XCDs x 32)
// Paged decode: the batch's KV tiles are cut into at most this many
// equal ranges (half as many for groups of 16 or more query heads), one wave
// each -- the waves one launch keeps resident on 256 CUs at eight per CU, so
// all of them start at once.
constexpr int kDecodeRanges = 2048;

struct DecodeArgs {
  const uint16_t* q;          // [B, H, D]
  const uint16_t* k_cache;    // [num_pages, 16, H_kv, D]
  const uint16_t* v_cache;
  const int32_t* page_table;  // [B, max_pages]
  const int32_t* seq_lens;    // [B]
  void* o;                    // [B, H, D], dtype of q or fp32 (out_f32)
  // Partials (workspace): [slots, rows_per_slot, D] and [slots,
  // rows_per_slot] (log2 domain), slot = work range + line; meta = {NT, W,
  // first tile of each sequence (B + 1 entries)}.
  float* part_o;
  float* part_lse;
  int* meta;
  int B, H, max_pages, n_splits;  // n_splits = the most work ranges
  int H_kv, group, qchunks;   // qchunks = ceil(group / 32)
  int min_tiles, rows_per_slot;  // tiles per range at least; min(group, 32)
  int num_pages;              // page ids outside [0, num_pages) are rejected on the device
  float c;                    // scale * log2(e)
};

hipError_t launch_paged_decode_gqa(int D, bool bf16, bool out_f32, const DecodeArgs& a,
                                   hipStream_t s);

// Argument checks of paged decode (api.cpp), shared by the entry point that
// takes a workspace and the one that uses the library's own array.
int check_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, const int32_t* seq_lens, const void* o, int B,
                       int H, int H_kv, int D, int page_size, int num_pages,
                       int max_pages_per_seq, int dtype, float scale, size_t* need);

}  // namespace mi355_attn
