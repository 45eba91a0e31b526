/*
 * attn.h -- C ABI of the MI355X (gfx950) fused-attention library.
 *
 * Scaled-dot-product attention
 *
 *     O[b,h,i,:] = sum_j softmax_j(scale * <q_i, k_j> + M_ij) * v_j
 *
 * as a flash-style prefill ("WAVE: A Symbolic Python DSL and Compiler for
 * High Performance Machine Learning (MLSys 2026)", core method, and its
 * attention experiments over BHSD and BSHD layouts) and as paged flash
 * decoding ("Wave February 2025 Release", FlashDecoding list), with grouped
 * KV heads, extend attention after a paged prefix, fp8 inputs, and the
 * backward pass of the prefill (roadmap items of the same release).
 *
 * Conventions for every entry point:
 *   - Every pointer is a device pointer owned by the caller.  The library never
 *     allocates, frees, synchronises, or reads device memory on the host, so
 *     every call is safe inside HIP graph capture.
 *   - Work is enqueued on `stream` (0 = the null stream) and is asynchronous;
 *     a kernel fault surfaces at the caller's next synchronisation.
 *   - Return codes are synchronous.  All argument checks run before any HIP
 *     call, so they also work on a host without a GPU.  After a launch,
 *     hipGetLastError() is mapped to ATTN_E_HIP.
 *   - Tensors are densely packed in the stated layout; outputs must not alias
 *     inputs; pointers are 16-byte aligned.
 */
#ifndef MI355_ATTN_H
#define MI355_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = 1,      /* null pointer, negative size, bad scale, misaligned pointer */
  ATTN_E_UNSUPPORTED = 2,  /* valid request the library does not implement (head dim, page size) */
  ATTN_E_WORKSPACE = 3,    /* workspace missing or smaller than the entry point's *_workspace_size */
  ATTN_E_HIP = 4           /* the HIP runtime reported an error at launch */
};

/* Memory layouts of q, k, v and o. */
enum {
  ATTN_BHSD = 0,  /* [B, H, S, D], D contiguous */
  ATTN_BSHD = 1   /* [B, S, H, D], D contiguous */
};

/* Element types of q, k, v, o (and of the KV cache).  ATTN_OUT_F32 may be
 * OR-ed into `dtype`: o is then fp32 (same shape and layout, 4-byte
 * elements) and receives the fp32 result before any rounding to fp16/bf16.
 * This is the higher-precision output of the same computation, for callers
 * that feed O on in fp32 or compare against a higher-precision reference
 * (grading against a higher-precision reference: "[FlyDSL] FP8 MQA logits
 * improvements for gfx950", Testing). */
enum {
  ATTN_F16 = 0,
  ATTN_BF16 = 1,
  ATTN_OUT_F32 = 0x100
};

/* Human-readable name of a status code (static storage; never NULL). */
const char* attn_status_string(int status);

/*
 * Fused scaled-dot-product attention prefill.
 *
 *   q: [B, H, Sq, D] (BHSD) or [B, Sq, H, D] (BSHD)
 *   k, v: the same with Skv keys
 *   o: output, same shape and layout as q; dtype as q, or fp32 with ATTN_OUT_F32
 *   D: head dimension, 64 or 128 (else ATTN_E_UNSUPPORTED)
 *   dtype: ATTN_F16 or ATTN_BF16 (q, k, v share it; o too unless
 *          ATTN_OUT_F32 is OR-ed in); any other bit is ATTN_E_INVALID
 *   causal: nonzero for the causal mask, aligned bottom-right: query i sees
 *           keys j <= i + (Skv - Sq).  A query that sees no key gets O = 0.
 *   scale: softmax scale, finite and >= 0 (commonly 1/sqrt(D)).
 *
 * Arithmetic: Q.K^T in the input dtype on MFMA with fp32 accumulation; the
 * online softmax in fp32 (base-2 exponent, scale folded in fp32, never into
 * the fp16/bf16 inputs); P rounded to fp16 (round to nearest even) and P.V on
 * fp16 MFMA with fp32 accumulation; O rounded to the input dtype (to
 * nearest even), or stored in fp32 with ATTN_OUT_F32.  For bf16
 * inputs V is converted to fp16 when it is staged, which is exact for
 * 2^-14 <= |v| <= 65504; precondition for bf16: |v| <= 65504.
 *
 * B, H, Sq or Skv equal to 0 is valid: with B*H*Sq = 0 nothing is launched and
 * q/k/v/o may be NULL; with Skv = 0 (and Sq > 0) o is filled with zeros.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o,
                 int B, int H, int Sq, int Skv, int D, int layout, int dtype,
                 int causal, float scale, hipStream_t stream);

/*
 * Grouped-query (and multi-query) prefill: as attn_prefill, with k and v
 * holding H_kv heads ([B, H_kv, Skv, D] or [B, Skv, H_kv, D]) shared by the H
 * query heads: query head h reads KV head h / (H / H_kv).  H_kv must divide H
 * (else ATTN_E_INVALID); H_kv = H is attn_prefill, H_kv = 1 multi-query
 * attention.  The pages do not define grouped heads; this is the mapping
 * that consecutive query heads share a KV head.  attn_prefill(...) is
 * attn_prefill_gqa(..., H, H, ...).
 */
int attn_prefill_gqa(const void* q, const void* k, const void* v, void* o,
                     int B, int H, int H_kv, int Sq, int Skv, int D, int layout, int dtype,
                     int causal, float scale, hipStream_t stream);

/*
 * attn_prefill_gqa that also stores each query row's log-sum-exp, for the
 * backward pass: lse [B, H, Sq] fp32 (BHSD order whatever the layout), the
 * natural log of sum_j exp(scale <q_i, k_j> + M_ij), -inf for a row with no
 * visible key.  lse may be NULL (then this is attn_prefill_gqa); it must be
 * 4-byte aligned.
 */
int attn_prefill_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int H_kv, int Sq, int Skv, int D, int layout, int dtype,
                     int causal, float scale, hipStream_t stream);

/*
 * attn_prefill_gqa for grids too small to fill the GPU (few query tiles
 * against many keys: chunked prefill, a short query block over a long
 * context): the keys of each query tile are split across workgroups, each
 * writing a partial output and log-sum-exp into the workspace, and a second
 * kernel merges them by log-sum-exp (flash decoding applied to prefill:
 * "Wave February 2025 Release", FlashDecoding list; the KV split sized to
 * fill the GPU: "[FlyDSL] FP8 MQA logits improvements for gfx950", Changes /
 * Host side).  The split count comes from sizes only
 * (attn_prefill_splitkv_num_splits); with one split (the grid already holds
 * two workgroups per CU, fewer than 1024 keys, or no split modelled faster)
 * this is attn_prefill_gqa,
 * needs no workspace and gives its result bitwise.  Otherwise the result is
 * attn_prefill_gqa's up to the rounding of the merge (the partials are fp32;
 * each split's P is rounded to fp16 as in attn_prefill).
 *
 *   workspace: device scratch of at least attn_prefill_splitkv_workspace_size
 *       bytes (0: may be NULL), 16-byte aligned, owned by the caller; its
 *       contents need no initialisation.  ATTN_E_WORKSPACE if missing or small.
 * Every other argument and error as in attn_prefill_gqa.
 */
int attn_prefill_splitkv(const void* q, const void* k, const void* v, void* o,
                         int B, int H, int H_kv, int Sq, int Skv, int D, int layout,
                         int dtype, int causal, float scale, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Key splits per query tile attn_prefill_splitkv uses for these sizes (1: no
 * split; 0 for invalid sizes).  Each split covers at least 512 keys; the
 * count is the one with the least modelled time on 256 CUs: the busiest CU's
 * workgroups times one key range's tiles, plus the fp32 partials of every
 * split at HBM rate.  Splits are considered only below two workgroups (query
 * tiles x heads x batch) per CU. */
int attn_prefill_splitkv_num_splits(int B, int H, int Sq, int Skv, int D);

/* Workspace bytes of attn_prefill_splitkv (0 when it does not split): per
 * split, fp32 partial outputs [B*H*Sq*D] and log-sum-exps [B*H*Sq], each
 * array padded to 256 bytes. */
size_t attn_prefill_splitkv_workspace_size(int B, int H, int Sq, int Skv, int D);

/* Workspace bytes of attn_prefill_bwd: two fp32 per query row (delta =
 * rowsum(dO * O) and -LSE log2(e)), each array padded to 256 bytes. */
size_t attn_prefill_bwd_workspace_size(int B, int H, int Sq);

/*
 * Backward of attn_prefill_gqa (backward flash attention: "Wave February 2025
 * Release" roadmap): the gradients dq, dk, dv of sum(O * dO) for
 * O = attention(q, k, v), by the chain rule with P recomputed from lse:
 *
 *   dV_j = sum_i P_ij dO_i,  dP_ij = <dO_i, V_j>,  delta_i = <dO_i, O_i>,
 *   dS_ij = P_ij (dP_ij - delta_i),
 *   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i,
 *
 * grouped heads summing into their KV head's dk, dv.
 *
 *   q, o, dO, dq: like q of attn_prefill_gqa; k, v, dk, dv: like k; lse: from
 *   attn_prefill_lse on the same inputs.  dq, dk, dv: the input dtype, or
 *   fp32 with ATTN_OUT_F32 in dtype.  Every row of dq, dk and dv is written.
 *   workspace: >= attn_prefill_bwd_workspace_size(B, H, Sq) bytes, 16-byte
 *   aligned, no initialisation needed.
 *
 * Arithmetic: S and dP on MFMA in the input dtype with fp32 accumulation; P
 * and dS rounded to the input dtype as MFMA operands; dO, Q, K, V used as
 * given.  Deterministic: no atomics (dk, dv are summed inside one workgroup,
 * dq by a second kernel).
 */
int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dO, const float* lse, void* dq, void* dk, void* dv,
                     int B, int H, int H_kv, int Sq, int Skv, int D, int layout, int dtype,
                     int causal, float scale, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * FP8 prefill: attn_prefill_gqa with q, k, v in OCP e4m3fn (one byte per
 * element, same shapes and layouts) and per-tensor descales: the inputs are
 * q_descale * Q, k_descale * K, v_descale * V.  (FP8 flash attention is a
 * roadmap item of "Wave February 2025 Release"; e4m3fn with per-tensor
 * scales is the format of the fp8 kernels in "[FlyDSL] FP8 MQA logits
 * improvements for gfx950".)
 *
 *   out_dtype: ATTN_F16 or ATTN_BF16 -- the type of o -- optionally OR-ed
 *              with ATTN_OUT_F32 (o in fp32)
 *   descales: finite and >= 0 (else ATTN_E_INVALID)
 *
 * Arithmetic: Q.K^T on the gfx950 fp8 MFMA (exact products, fp32
 * accumulation) with scale * q_descale * k_descale * log2(e) folded in fp32
 * into the exponent; P rounded to fp16 and P.V on fp16 MFMA with V widened
 * e4m3fn -> fp16 (exact) on staging; O = v_descale * (P.V) / l.
 */
int attn_prefill_fp8(const void* q, const void* k, const void* v, void* o,
                     int B, int H, int H_kv, int Sq, int Skv, int D, int layout, int out_dtype,
                     int causal, float scale, float q_descale, float k_descale, float v_descale,
                     hipStream_t stream);

/*
 * Extend attention: prefill of new tokens after a cached prefix (chunked
 * prefill; the "extend" call of an LLM serving backend: "WAVE: A Symbolic
 * Python DSL and Compiler for High Performance Machine Learning (MLSys 2026)",
 * integration notes; extend attention in the "Wave February 2025 Release"
 * roadmap).  For each of the B sequences:
 *
 *   - prefix_lens[b] tokens are already in a paged cache k_cache, v_cache
 *     [num_pages, page_size, H_kv, D], token t at page page_table[b][t / 16],
 *     slot t % 16 (page_table [B, max_pages_per_seq] int32), as in
 *     attn_paged_decode_gqa;
 *   - its E_b = qo_start[b+1] - qo_start[b] new tokens are rows qo_start[b] ..
 *     qo_start[b+1]-1 of q [total_tokens, H, D], k, v [total_tokens, H_kv, D]
 *     and o [total_tokens, H, D] (packed token-major; qo_start [B+1] int32);
 *   - new token i attends to every prefix token and to new tokens 0..i
 *     (causal attention over prefix + new tokens, aligned bottom-right), query
 *     head h to KV head h / (H / H_kv).
 *
 * The pages do not define the operation further; this is the plain reading
 * (the new tokens' K/V are not written to the cache here).  max_extend_len
 * >= every E_b bounds the grid: rows of a sequence past max_extend_len are
 * not written.  page_size: 16; D: 64 or 128.  Arithmetic as attn_prefill.
 * Key positions are 32-bit: max_pages_per_seq * 16 + max_extend_len must be
 * below 2^31, and max_extend_len * H * D * 2 (a sequence's rows of q in
 * bytes) too (else ATTN_E_UNSUPPORTED).
 *
 * Device data (read only on the device): prefix_lens[b] is clamped to
 * [0, max_pages_per_seq * 16]; a sequence whose qo_start range is not within
 * [0, total_tokens] is skipped (its rows are not written); a prefix page id
 * outside [0, num_pages) is never dereferenced and makes the sequence's rows
 * NaN.  With max_pages_per_seq = 0 there is no prefix and k_cache, v_cache,
 * page_table and prefix_lens may be NULL.
 */
int attn_extend(const void* q, const void* k, const void* v,
                const void* k_cache, const void* v_cache,
                const int32_t* page_table, const int32_t* prefix_lens, const int32_t* qo_start,
                void* o, int B, int H, int H_kv, int D, int total_tokens, int max_extend_len,
                int page_size, int num_pages, int max_pages_per_seq, int dtype, float scale,
                hipStream_t stream);

/*
 * attn_extend for grids too small to fill the GPU (few sequences and new
 * tokens after long cached prefixes: chunked prefill of one long prompt
 * through the paged cache): each unit's keys (its prefix tiles, then its new
 * tokens' tiles) are split across workgroups, each writing a partial output
 * and log-sum-exp into the workspace, and a second kernel merges them by
 * log-sum-exp (flash decoding applied to extend: "Wave February 2025
 * Release", FlashDecoding list and Extend Attention, split-k; the KV split
 * sized to fill the GPU: "[FlyDSL] FP8 MQA logits improvements for gfx950",
 * Changes / Host side).  The split count comes from sizes only
 * (attn_extend_splitkv_num_splits, from the bounds max_extend_len and
 * max_pages_per_seq * 16); with one split this is attn_extend, needs no
 * workspace and gives its result bitwise.  Otherwise the result is
 * attn_extend's up to the rounding of the merge, and the rows written are
 * the same: rows of sequences whose qo_start range is invalid, and rows past
 * max_extend_len, are not written; a rejected prefix page makes the
 * sequence's rows NaN.
 *
 *   workspace: device scratch of at least attn_extend_splitkv_workspace_size
 *       bytes (0: may be NULL), 16-byte aligned, owned by the caller; its
 *       contents need no initialisation.  ATTN_E_WORKSPACE if missing or small.
 * Every other argument and error as in attn_extend.
 */
int attn_extend_splitkv(const void* q, const void* k, const void* v,
                        const void* k_cache, const void* v_cache,
                        const int32_t* page_table, const int32_t* prefix_lens,
                        const int32_t* qo_start, void* o, int B, int H, int H_kv, int D,
                        int total_tokens, int max_extend_len, int page_size, int num_pages,
                        int max_pages_per_seq, int dtype, float scale, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Key splits per unit attn_extend_splitkv uses for these sizes (1: no split,
 * also when there is nothing to compute; 0 for invalid sizes), by the model
 * of attn_prefill_splitkv_num_splits over attn_extend's grid: units of
 * max_extend_len new tokens after max_pages_per_seq * 16 prefix tokens. */
int attn_extend_splitkv_num_splits(int B, int H, int H_kv, int D, int total_tokens,
                                   int max_extend_len, int max_pages_per_seq);

/* Workspace bytes of attn_extend_splitkv (0 when it does not split): per
 * split, fp32 partial outputs [total_tokens*H*D] and log-sum-exps
 * [H*total_tokens], each array padded to 256 bytes. */
size_t attn_extend_splitkv_workspace_size(int B, int H, int H_kv, int D, int total_tokens,
                                          int max_extend_len, int max_pages_per_seq);

/*
 * Bytes of device workspace attn_paged_decode needs for these sizes: the
 * partial outputs and log-sum-exps of the work ranges, and the ranges'
 * metadata.  Returns 0 for invalid sizes.
 */
size_t attn_paged_decode_workspace_size(int B, int H, int D, int max_pages_per_seq,
                                        int page_size);

/*
 * Split-KV paged flash decoding: one query per sequence against a paged KV cache.
 *
 *   q: [B, H, D]
 *   k_cache, v_cache: [num_pages, page_size, H, D]; token t of sequence b is
 *       at page page_table[b][t / page_size], slot t % page_size
 *   page_table: [B, max_pages_per_seq] int32
 *   seq_lens: [B] int32
 *   o: [B, H, D] output, dtype as q, or fp32 with ATTN_OUT_F32 in dtype
 *   page_size: 16 (else ATTN_E_UNSUPPORTED); D: 64 or 128
 *   workspace: device scratch of at least
 *       attn_paged_decode_workspace_size(B, H, D, max_pages_per_seq, page_size)
 *       bytes, owned by the caller; its contents need no initialisation.
 *
 * Device data (read only on the device; the host never sees it):
 *   - seq_lens[b] is clamped to [0, max_pages_per_seq * page_size]; a
 *     sequence of length 0 (or less) gets O = 0.
 *   - The first ceil(seq_lens[b] / page_size) entries of page_table[b] are
 *     checked on the device before any load through them: an id outside
 *     [0, num_pages) is never dereferenced, and O[b] (every head) is NaN.
 *   - Other page-table entries and cache slots past seq_lens[b] are never read.
 *
 * Flash decoding ("Wave February 2025 Release", FlashDecoding list): the
 * batch's KV is cut into pieces, each producing a partial output and its
 * log-sum-exp, and a combine kernel merges them.  The pieces are equal work
 * ranges of the batch's 32-token tiles, cut on the device from the actual
 * lengths (sized to fill the GPU: "[FlyDSL] FP8 MQA logits improvements for
 * gfx950", Changes / Host side); see attn_paged_decode_gqa for the details
 * and the arithmetic, which are the same (this is attn_paged_decode_gqa with
 * H_kv = H).
 */
int attn_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* page_table, const int32_t* seq_lens, void* o,
                      int B, int H, int D, int page_size, int num_pages,
                      int max_pages_per_seq, int dtype, float scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Grouped-query (and multi-query) paged decode: as attn_paged_decode, with a
 * cache of H_kv heads ([num_pages, page_size, H_kv, D]) shared by the H query
 * heads of q: query head h reads KV head h / (H / H_kv).  H_kv must divide H
 * (else ATTN_E_INVALID).  The query heads of a group are decoded together,
 * so each cache row is read from memory once per group; with H_kv = H this
 * is attn_paged_decode.  The workspace comes from
 * attn_paged_decode_gqa_workspace_size; page ids and lengths are treated as
 * in attn_paged_decode (a bad page id makes O[b] NaN for every head).
 * Arithmetic: Q.K^T on MFMA in the input dtype with fp32 accumulation,
 * softmax in fp32, P rounded to fp16 and P.V on fp16 MFMA (bf16 V converted
 * to fp16 on staging, as in attn_prefill).
 * Work division: the batch's 32-token tiles, taken sequence by sequence and
 * KV head by KV head, are cut on the device into W equal contiguous ranges
 * (W at most attn_paged_decode_gqa_num_splits, fewer for short batches), one
 * wave each; a range that crosses sequences writes one partial per sequence
 * and KV head it touches, and the log-sum-exp combine merges them.  The
 * workspace also holds the range metadata, rewritten by every call.  With
 * fp16 inputs and fp16 output the partial outputs (normalised, so within
 * fp16 range) are kept in fp16; otherwise in fp32.
 */
int attn_paged_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* page_table, const int32_t* seq_lens, void* o,
                          int B, int H, int H_kv, int D, int page_size, int num_pages,
                          int max_pages_per_seq, int dtype, float scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): paged
 * decode as attn_paged_decode_gqa -- same arguments without the workspace,
 * same kernels, bitwise the same results and device-side checks -- with the
 * partial results kept in a device array the library owns:
 * ATTN_DECODE_SCRATCH_BYTES (32 MiB) on each GPU the library runs on,
 * reserved when the library's device code is loaded there and held until the
 * process ends.  Nothing is allocated, freed or synchronised by the call.
 *
 *   - Sizes whose attn_paged_decode_gqa_workspace_size exceeds
 *     ATTN_DECODE_SCRATCH_BYTES are refused with ATTN_E_WORKSPACE, after the
 *     other argument checks and before any HIP call.
 *   - The array needs no initialisation: every call writes each partial and
 *     the metadata it reads back.  It keeps the last call's contents.
 *   - Every call on one GPU uses that GPU's single array: calls that may
 *     overlap on one GPU (other streams, other host threads) race on it, and
 *     the caller must order them (for example, one stream per GPU).
 *   - The first call on a device looks the array's address up on the device
 *     current at that call (hipGetSymbolAddress, no allocation); ATTN_E_HIP if
 *     the runtime cannot give it.  `stream` must belong to the current device
 *     (else ATTN_E_INVALID).
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int attn_paged_decode_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* page_table, const int32_t* seq_lens, void* o,
                                  int B, int H, int H_kv, int D, int page_size, int num_pages,
                                  int max_pages_per_seq, int dtype, float scale,
                                  hipStream_t stream);

/* Workspace bytes of attn_paged_decode_gqa (0 for invalid sizes). */
size_t attn_paged_decode_gqa_workspace_size(int B, int H, int H_kv, int D,
                                            int max_pages_per_seq, int page_size);

/* Work plan of attn_paged_decode_gqa: returns the largest number of work
 * ranges W a call uses (0 on invalid sizes) and, if tokens_per_split is not
 * NULL, stores there the fewest tokens a range covers unless the batch holds
 * fewer: 16 per query head of the group, at most 256, at least 128.  W is at
 * most 2048, or 1024 for groups of 16 or more query heads.  The plan depends
 * only on these host-side sizes (the host never reads seq_lens); the ranges
 * themselves are cut on the device from the actual lengths. */
int attn_paged_decode_gqa_num_splits(int B, int H, int H_kv, int max_pages_per_seq,
                                     int page_size, int* tokens_per_split);

/* Work plan of attn_paged_decode: attn_paged_decode_gqa_num_splits with
 * H_kv = H. */
int attn_paged_decode_num_splits(int B, int H, int max_pages_per_seq, int page_size,
                                 int* tokens_per_split);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ATTN_H */
