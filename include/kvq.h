/*
 * kvq.h -- C ABI of libkvq: quantize-on-write into a paged INT8 KV cache, split-KV
 * grouped-query decode attention over that cache, and the log-sum-exp merge, for one
 * AMD Instinct MI355X (gfx950).
 *
 * The operations and where they are defined:
 *   kvq_write            quantize-on-write.  Half-the-memory page ("Making a ternary
 *                        reasoning model fast in vLLM", anthonymorley.com), section "Is 8 bits
 *                        enough?": llama.cpp's Q8_0 cache format, one scale per 32 values;
 *                        gllm page (git.kenbook.uk/GlowLED/gllm), section "Quantization
 *                        Design": symmetric int8, scale amax/127, round to nearest, clamp to
 *                        +-127, dynamic per token; NVFP4 page (dev.to, "Building an NVFP4 KV
 *                        cache ..."), section "Writing and reading the packed cache": BF16
 *                        values plus a token-to-slot map, invalid slots do not write, valid
 *                        slots unique within a call.
 *   kvq_decode_attention split-KV decode attention and merge.  Long-context page ("long
 *                        context attention and lessons", anthonymorley.com), section "Give more
 *                        GPU workers a piece of the attention calculation": segments of the
 *                        context computed in parallel, each giving a weighted value sum and its
 *                        normalisation terms, combined with those terms; half-the-memory page,
 *                        section "Read the compressed cache without copying it first": one
 *                        query token reads the int8 cache directly, V dequantized in registers,
 *                        no converted copy of the cache.
 *   kvq_decode_attention_mq  several query tokens per sequence (multi-token decode, for example
 *                        checking drafted tokens), causal among them.  Half-the-memory page, section
 *                        "The stock path was slow" and the request-performance sections: steps
 *                        that generate or check up to 16 tokens per request run on the INT8
 *                        kernel; each query token attends to the cache up to its own position.
 *   kvq_decode_step      one decode step of one layer in a single kernel pass: the new token's
 *                        quantize-on-write (as kvq_write) fused into the split kernel, then the
 *                        merge (as kvq_decode_attention).  Gllm page, section "Interpretation":
 *                        at decode batch sizes the extra quantize launches per layer cost more
 *                        than the quantization saves; section "Known Limitations": graph capture
 *                        breaks when a kernel of the step allocates (the step allocates nothing).
 *   kvq_check_write,     checked wrappers.  NVFP4 page, section "Testing the cache without
 *   kvq_check_decode,    loading the model": a checked API that validates on the host,
 *   kvq_check_decode_step synchronises, and refuses graph capture; raw callers own stream
 *                        ordering and cache lifetime.
 *
 * Arithmetic.  kvq_write: x = float(bf16); amax = max |x| over 32 consecutive channels of one
 * (token, KV head); d = amax / 127 (IEEE fp32 division); s = fp16(min(d, 65504)), round to
 * nearest even, stored; code = clamp(rint(x / s), -127, 127) in fp32 with ties to even
 * (x / s the correctly rounded quotient), 0 when s == 0.  The decoded value is code * s.  kvq_decode_attention returns, per sequence s
 * and query head hq (KV head h = hq / (Hq / Hkv)):
 *   out[s][hq][:] = sum_t softmax_t(q . k_t / sqrt(D)) v_t   over t < context_lens[s]
 *   lse[s][hq]    = ln sum_t exp(q . k_t / sqrt(D))            (natural log)
 * computed with fp32 accumulation; an empty context gives out = 0 and lse = -inf.
 *
 * Cache layout (one kvq_cache_t per layer, all buffers owned by the caller, device memory):
 *   INT8 (KVQ_INT8_Q8_0):
 *     k, v           int8, num_blocks * Hkv pages of 16*D bytes, page (block b, KV head h)
 *                    at byte offset (b*Hkv + h) * 16*D.  Inside a page the byte of token t
 *                    (0..15) and channel c (0..D-1) is at
 *                      K:  ((((c>>6)<<6) | (((c>>3)&3)<<4) | t) << 4) | (((c>>5)&1)<<3) | (c&7)
 *                      V:  ((((c>>6)<<6) | ((t>>2)<<4) | (c&15)) << 4) | (((c>>4)&3)<<2) | (t&3)
 *                    (kvq_page_offset() returns the same values).
 *     k_scales,      binary16, [num_blocks][Hkv][D/32][16]: scale of (token t, group g = c/32)
 *     v_scales       at element ((b*Hkv + h)*(D/32) + g)*16 + t (group-major within a page, so
 *                    that the 4 scales of one group a lane needs are 8 contiguous bytes).
 *   INT8 per head (KVQ_INT8_PER_HEAD): the half-the-memory page's description of vLLM's
 *     int8_per_token_head cache (one shared 32-bit scale per token and head; 520 bytes per token
 *     per head at D = 256): k, v codes exactly as for KVQ_INT8_Q8_0; k_scales, v_scales fp32
 *     [num_blocks][Hkv][16], element (b*Hkv + h)*16 + t.  Quantizer: amax over the row's D values,
 *     s = amax / 127 (fp32 division, stored as is), code = clamp(rint(x / s), -127, 127) with the
 *     fp32 quotient rounded half to even, 0 when s == 0.
 *   BF16 (KVQ_BF16):  k, v bfloat16, pages of 16*D values (2*16*D bytes); element of (t, c):
 *                      K:  (((c>>5)<<6) | (((c>>3)&3)<<4) | t) << 3 | (c&7)
 *                      V:  (((c>>5)<<6) | ((t>>2)<<4) | (c&15)) << 3 | (((c>>4)&1)<<2) | (t&3)
 *                    k_scales = v_scales = NULL.
 *   A slot is block*16 + offset; token t of sequence s is in slot
 *   block_tables[s][t/16]*16 + t%16.  Every plane base must be 256-byte aligned.
 *   Supported: block_size 16, head_dim 128 or 256, Hq % Hkv == 0, 1 <= Hq/Hkv <= 16.
 *
 * Errors.  Every entry point returns kvq_status_t (0 = KVQ_OK).  Host-side checks of
 * scalars and pointers run before anything is enqueued; on error nothing is launched.
 * No C++ exception crosses this interface.  The fast paths never allocate, free or
 * synchronise and are safe to capture into a HIP graph.  The library writes only: the
 * (slot, head) rows of valid slots in the cache, out, lse and the workspace.
 *
 * Streams are hipStream_t passed as void* (NULL = the default stream).  Device pointers
 * are plain device addresses on the current HIP device.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_INT8_Q8_0 = 0,    /* int8 codes + one binary16 scale per 32 values */
  KVQ_BF16 = 1,         /* bfloat16 values, no scales (comparison variant) */
  KVQ_INT8_PER_HEAD = 2 /* int8 codes + one fp32 scale per (token, KV head) row (comparison format) */
} kvq_dtype_t;

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1,         /* null/misaligned pointer, bad count or dimension */
  KVQ_ERR_UNSUPPORTED = -2,         /* head_dim, block_size, dtype or GQA ratio not supported */
  KVQ_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes below kvq_decode_workspace_bytes() */
  KVQ_ERR_LAUNCH_FAILED = -4,       /* the HIP runtime reported an error */
  KVQ_ERR_VALIDATION_FAILED = -5,   /* checked mode: device data broke the contract */
  KVQ_ERR_CAPTURING = -6            /* checked mode called during stream capture */
} kvq_status_t;

typedef struct {
  int32_t dtype;        /* kvq_dtype_t */
  int32_t num_blocks;   /* pages per KV head in the pool */
  int32_t block_size;   /* tokens per page; must be 16 */
  int32_t num_kv_heads; /* Hkv: 1 .. 65535 */
  int32_t head_dim;     /* D: 128 or 256 */
  void *k, *v;          /* code / value planes (layout above) */
  void *k_scales, *v_scales; /* scale planes: binary16 (q8_0) or fp32 (per head); NULL for BF16 */
} kvq_cache_t;

/*
 * Quantize-on-write (INT8) or scatter copy (BF16) of num_tokens new tokens.
 *   k, v          device, bfloat16 [num_tokens][Hkv][D], contiguous, 16-byte aligned.
 *   slot_mapping  device, int32 [num_tokens]; slot < 0 (or >= num_blocks*16): not written.
 * Valid slots must be unique within one call (caller's contract; the fast path does not
 * check it).  Writing a slot replaces every code and scale of that (slot, head) row.
 * num_tokens == 0 is a no-op.  Asynchronous on `stream`.
 * Fewer than 16 tokens (a decode batch's step) are written by one thread per 32-value group
 * (BF16: per 8 values; per-head format: one wavefront per row).  From 16 tokens on, each
 * workgroup takes 16 consecutive tokens of the call; a run of 16 tokens whose slots fill one
 * page in order (as a prefill writes them) is stored as whole page rows.  Results are the same
 * byte for byte either way.
 */
int kvq_write(const kvq_cache_t *cache, const void *k, const void *v, const int32_t *slot_mapping,
              int32_t num_tokens, void *stream);

/*
 * Bytes of workspace kvq_decode_attention needs for these sizes; num_splits is the split
 * count actually used (1..4096; for the automatic choice pass kvq_choose_num_splits()'s
 * result).  The workspace holds what each segment of the context hands to the combination step
 * (long-context page, section "Give more GPU workers a piece of the attention calculation": a
 * weighted value sum and its normalisation terms per segment): fp32 weighted sums
 * [S][Hq][splits][D] (256-byte aligned) followed by (max, sum) pairs [S][Hq][splits][2].
 * Returns 0 on invalid arguments.
 */
size_t kvq_decode_workspace_bytes(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_splits);

/*
 * Split count the library uses when kvq_decode_attention gets num_splits == 0.  Long-context
 * page, section "Split count": the best number of segments depends on the context length and is
 * found by sweeping it; section "Give more GPU workers a piece of the attention calculation":
 * segments exist to give every compute unit work.  Here: enough workgroups to fill the device's
 * compute units, no segment shorter than 8 pages, from sweeps on 256 CUs.  Depends only on the
 * host-side sizes and the device's compute-unit count (no device synchronisation).  Returns a
 * negative kvq_status_t on invalid arguments.
 */
int32_t kvq_choose_num_splits(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_context_len);

/*
 * Split count from the batch's actual context lengths, for callers that hold them on the host
 * (the same sources as kvq_choose_num_splits: segments give every compute unit work, and their
 * best number depends on the lengths).  The decode kernels cut every sequence into segments of
 * the same length, max_context_len / num_splits, so a sequence shorter than the maximum fills
 * only part of its segments; kvq_choose_num_splits sees only the maximum and cannot tell a
 * batch of equal lengths from a ragged one.  Here, for a batch with fewer (sequence, KV head)
 * pairs than compute units, the segment length is chosen so that the non-empty segments make
 * about four rounds of the compute units (a multiple of 4 pages, at least 8); otherwise (one
 * sequence, or many pairs) the result is kvq_choose_num_splits(max length).  Pass it as
 * num_splits (and to kvq_decode_workspace_bytes).
 *   host_context_lens  host, int32 [num_seqs], each >= 0 (the lengths the decode will see).
 * Returns 1..4096, or a negative kvq_status_t on invalid arguments (a null array, a negative
 * length).  Reads nothing on the device.
 */
int32_t kvq_choose_num_splits_lengths(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_q_heads,
                                      const int32_t *host_context_lens);

/*
 * Split-KV decode attention for one query token per sequence, then the merge.
 *   q                  device, bfloat16 [num_seqs][num_q_heads][D], 16-byte aligned.
 *   block_tables       device, int32 [num_seqs][max_blocks_per_seq].
 *   context_lens       device, int32 [num_seqs]; tokens 0..context_lens[s]-1 are attended
 *                      (the token written by this step's kvq_write included); must satisfy
 *                      0 <= context_lens[s] <= max_context_len.  A length of 0 (a slot of the
 *                      batch with no tokens yet) is accepted and gives out = 0, lse = -inf.
 *   max_context_len    host: upper bound of context_lens, sizes the grid without a sync;
 *                      1 <= max_context_len <= max_blocks_per_seq*16.
 *   num_splits         0 = automatic (kvq_choose_num_splits), else 1..4096.
 *   out                device, fp32 [num_seqs][num_q_heads][D].
 *   lse                device, fp32 [num_seqs][num_q_heads], or NULL.
 *   workspace          device, at least kvq_decode_workspace_bytes(...) bytes, 256-byte
 *                      aligned; its contents on entry do not matter.
 * Context lengths and block ids outside the contract are clamped for memory safety (the
 * result is then unspecified, no fault).  Asynchronous on `stream`.
 */
int kvq_decode_attention(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode attention for num_query_tokens (n_q, 1..65536) query tokens per sequence, causal among
 * them (INT8 caches).  Large n_q is a prompt section over the cache: half-the-memory page,
 * section "Read the prompt using a small temporary buffer": a new prompt section attends to the
 * cached keys before it and causally to itself, the parts combined with their attention weights;
 * here straight from the INT8 pages (no converted copy), the combination being the split merge.
 * The query tokens of sequence s are its last n_q positions L-n_q .. L-1 (L = context_lens[s],
 * which includes them): query token i attends to the keys at positions 0 .. L-n_q+i.  n_q == 1
 * is kvq_decode_attention.
 *   q            device, bfloat16 [num_seqs][n_q][num_q_heads][D], 16-byte aligned.
 *   out          device, fp32 [num_seqs][n_q][num_q_heads][D].
 *   lse          device, fp32 [num_seqs][n_q][num_q_heads], or NULL.
 *   workspace    at least kvq_decode_workspace_bytes(cache, num_seqs * n_q, num_q_heads, splits)
 *                bytes, where splits is num_splits or, for 0, kvq_choose_num_splits_mq(...).
 *   other arguments as kvq_decode_attention.  A query token with no visible key (L < n_q) gets
 *   out = 0 and lse = -inf.  Returns KVQ_ERR_UNSUPPORTED for a BF16 cache with n_q > 1.
 * The (query token, head) pairs of one KV head form the rows of 16-row MFMA tiles; up to 4
 * tiles (64 rows, 64 / G query tokens) share one workgroup and one read of each page.  Longer
 * runs are cut into chunks of 64 / G query tokens, each chunk attending over the keys up to its
 * own last token, so each chunk reads its prefix once.  One sequence's q block and partials must
 * stay below 2 GiB (n_q * Hq * D * 2 and n_q * Hq * splits * D * 4 bytes), else
 * KVQ_ERR_INVALID_ARG.
 */
int kvq_decode_attention_mq(const kvq_cache_t *cache, const void *q, int32_t num_query_tokens,
                            const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                            float *out, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kvq_decode_attention with integer Q.K (opt-in; INT8 q8_0 cache only, else KVQ_ERR_UNSUPPORTED).
 * Half-the-memory page, section "Read the compressed cache without copying it first": Q is
 * quantized to int8 once, like the cache (one fp16 scale per 32 values, codes against the stored
 * scale), and Q.K runs as integer dot products on the int8 keys (v_mfma_i32_16x16x32_i8), each
 * 32-channel group's exact int32 sum scaled by its Q and K scales.  The result is attention with
 * the quantized query: it differs from kvq_decode_attention by the query's rounding.  The page
 * reports 1.4-2.1% on its model; on the synthetic workloads, whose queries carry x20 outlier
 * channels, the relative L2 difference is about 9%.  Off by default for that reason.  Same
 * arguments and workspace as kvq_decode_attention.
 */
int kvq_decode_attention_int8qk(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                                int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out, float *lse,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Split count kvq_decode_attention_mq uses for num_splits == 0 (negative status on error).
 * Half-the-memory page, section "Read the compressed cache without copying it first": the pages
 * tune the split count (segments) for verification separately from one-token decode; long-context
 * page, section "Split count": it depends on the context length.  The rule is the one-token rule
 * (enough workgroups to cover the compute units, at least 8 pages per split) counted in the
 * workgroups this path launches, each holding up to 4 row tiles of (query token, head) pairs.  The
 * compute units' workgroup slots are counted as: one per CU for a q8_0 single chunk of 3 or 4 row
 * tiles (6 to 10 tokens at 6 query heads per KV head: one 8-wave workgroup fills a CU), three for
 * q8_0 prompt sections (which also get at least four rounds of workgroups), two for the other
 * workgroups of 3 or 4 tiles, and one otherwise.  Arguments as kvq_decode_attention_mq.
 */
int32_t kvq_choose_num_splits_mq(const kvq_cache_t *cache, int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t num_q_heads, int32_t max_context_len);

/*
 * One decode step: writes the new token of every sequence into the cache, then attention and
 * merge over the context that includes it.  The result equals kvq_write(k_new, v_new,
 * slot_mapping) followed by kvq_decode_attention(...) on the same stream, with slot_mapping[s]
 * the slot of token context_lens[s]-1 (block_tables[s][(L-1)/16]*16 + (L-1)%16); cache bytes,
 * out and lse are the same.  The workgroup that reads a sequence's last page (for one KV head)
 * writes the token into it before reading it, so no separate write kernel runs.
 *   k_new, v_new   device, bfloat16 [num_seqs][Hkv][D], contiguous, 16-byte aligned: the token
 *                  at position context_lens[s]-1 of each sequence.
 *   other arguments as kvq_decode_attention (same workspace size).
 * A sequence with context_lens[s] == 0 writes nothing; nothing is written when the block of the
 * last page is outside [0, num_blocks), nor when context_lens[s] > max_context_len (outside the
 * contract: the context is then cut at max_context_len for memory safety, and the token, whose
 * position lies past the cut, is not written anywhere).  Contract (checked by kvq_check_decode_step): the block
 * that receives a sequence's new token is not used by any other sequence of the call, and not
 * twice in that sequence's table (blocks shared between sequences hold only older tokens).
 * Asynchronous on `stream`; allocates nothing.
 */
int kvq_decode_step(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                    const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                    int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                    float *out, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kvq_decode_step for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace.  The split partials go to a fixed device buffer inside the library, one per device,
 * of kvq_decode_step_noalloc_max_bytes() bytes (8 MiB), held from the first call on that device
 * until the process ends.  A call whose partials would not fit (kvq_decode_workspace_bytes() with
 * the split count used, num_splits or the automatic choice, above that size) returns
 * KVQ_ERR_WORKSPACE_TOO_SMALL with nothing enqueued.  Allocates nothing (no hipMalloc, hipFree or
 * allocating library call).  The buffer is shared by every call on the device: calls that overlap
 * in time on one device (different streams, or host threads without ordering) race and give
 * unspecified results.  Results equal kvq_decode_step's with the same split count.
 */
int kvq_decode_step_noalloc(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                            const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                            float *out, float *lse, void *stream);

/* Size in bytes of the fixed device buffer kvq_decode_step_noalloc uses. */
size_t kvq_decode_step_noalloc_max_bytes(void);

/*
 * The two halves of kvq_decode_attention, for callers that combine partials themselves
 * (for instance partials of one sequence computed in several places) or time the split
 * kernel alone.  kvq_decode_partials writes, for every split that holds pages, the
 * unnormalised weighted value sum and its (max, sum) normalisation terms into the workspace
 * (long-context page, section "Give more GPU workers a piece of the attention calculation");
 * kvq_decode_merge combines them with those terms into out and lse.  Both take the same
 * sizes as kvq_decode_attention and must agree on num_splits (0 resolves the same way in
 * both) and max_context_len.
 */
int kvq_decode_partials(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, void *workspace,
                        size_t workspace_bytes, void *stream);
int kvq_decode_merge(const kvq_cache_t *cache, const int32_t *context_lens, int32_t max_context_len,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, const void *workspace,
                     size_t workspace_bytes, float *out, float *lse, void *stream);

/*
 * Checked mode (tests and debugging; not for hot loops).  Copies the metadata (and the bf16
 * inputs) to the host, synchronises `stream`, rejects contract violations with
 * KVQ_ERR_VALIDATION_FAILED before launching, then runs the fast path and synchronises
 * again.  kvq_check_write rejects duplicate valid slots, slots >= num_blocks*16 and
 * non-finite K/V.  kvq_check_decode rejects context_lens outside [0, max_context_len],
 * block ids outside [0, num_blocks) in the pages a sequence uses, and non-finite Q;
 * kvq_check_decode_step also non-finite new K/V and a block that receives a new token while
 * another sequence (or another page of the same one) uses it.  All refuse to run while `stream`
 * is being captured (KVQ_ERR_CAPTURING).
 */
int kvq_check_write(const kvq_cache_t *cache, const void *k, const void *v, const int32_t *slot_mapping,
                    int32_t num_tokens, void *stream);
int kvq_check_decode(const kvq_cache_t *cache, const void *q, const int32_t *block_tables,
                     int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t max_context_len,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_splits, float *out, float *lse,
                     void *workspace, size_t workspace_bytes, void *stream);
int kvq_check_decode_step(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q,
                          const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                          int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, int32_t num_splits,
                          float *out, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* In-page offset (bytes for INT8, elements for BF16) of (token 0..15, channel c) in a K
 * (which = 0) or V (which = 1) page, per the layout above; -1 on invalid arguments. */
int32_t kvq_page_offset(int32_t dtype, int32_t head_dim, int32_t which, int32_t token, int32_t channel);

/* Human-readable name of a kvq_status_t. */
const char *kvq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
